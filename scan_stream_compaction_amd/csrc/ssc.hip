// Single-pass scan, stream compaction and stable partition for MI355X
// (gfx950, CDNA4): HIP kernels and the C ABI declared in include/ssc.h.
//
// Method ("Day 33 compaction.cu", header comment; "CUDA Handbook ch. 13,
// Stream Compaction", Listings 13-17/13-18): flag each element with a
// predicate, exclusive-scan the flags, scatter survivors to out[rank]; the
// count is the top of the scan, and a partition sends rejected x[i] to
// out[K + i - rank[i]]. The whole path is one kernel launch over tiles whose
// numbers come from an atomic counter; each tile finds the number of
// survivors before it by a decoupled look-back over per-tile descriptors.
//
// MI355X-first tile shape. A same-address device-scope atomic is serialised
// across the 8 XCDs at roughly 11-12 ns, so a tile number is claimed once per
// 30720 elements (120 KiB). Workgroups are 1024 threads: 15 data wavefronts
// + 1 control wavefront that walks the look-back (its waits cannot share a
// wavefront with outstanding data loads, whose completions count in the same
// in-order counter). The compaction and partition kernel is persistent, one
// workgroup per compute unit, with each data wavefront holding its chunk of
// the current tile and, in flight, its chunk of the next: every tile's
// aggregate is published as soon as its data has landed, the loads of later
// tiles overlap the look-back waits, and survivors leave as contiguous runs
// staged in LDS. Ranks inside a wavefront come from packed DPP scans of the
// lanes' per-load flag counts. The kernel is a template over element formats
// (32-bit values, a caller's flag bytes, key-value pairs, 64-bit values) that
// share this pipeline. The scan of values runs in the same pipeline
// (scan_persistent_kernel), each chunk parked in LDS until the next tile's
// barrier hands over its base; between one and two tiles per compute unit a
// one-tile-per-workgroup kernel (scan_kernel: two rounds of 15 chunks, the
// last data wavefront to finish scanning the 30 chunk totals) is faster.
//
// Scratch needs no clearing between calls: tile numbers and an epoch come
// from one 64-bit atomic word {epoch:32 | next tile:32}, reset and advanced
// by the call itself (by its last claim where a call makes a known number of
// claims, else by the last workgroup to finish claiming), and descriptors
// carry the epoch as a tag. The counting passes reset their own
// accumulators (the last workgroup to finish does it).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "ssc.h"
#include "ssc_device.h"

namespace ssc {

// ------------------------------------------------------------ tile shape ---
// Streaming kernels (copy, counting, unordered comparison): a 512-thread
// workgroup (8 wavefronts) handles a sub-tile of 8192 elements, each
// wavefront 1024 consecutive ones with four 128-bit loads per lane.
constexpr int kBlock = 512;
constexpr int kWaves = kBlock / kWave;         // 8
constexpr int kLoads = 4;                      // 128-bit loads per lane per chunk
constexpr int kChunk = kWave * kLoads * 4;     // 1024 elements per wavefront chunk
constexpr int kSub = kBlock * kLoads * 4;      // 8192 elements per streaming sub-tile

// Look-back kernels (compaction, partition, scan): a 1024-thread workgroup =
// 15 data wavefronts + 1 control wavefront. The control wavefront claims the
// tile and walks the look-back while the data wavefronts load and rank; a
// tile is 2 rounds of 15 chunks (30720 elements, 120 KiB), 32 elements per
// data lane from eight 128-bit loads.
constexpr int kLbBlock = 1024;
constexpr int kDataWaves = 15;
constexpr int kCtrlWave = 15;                  // index of the control wavefront
constexpr int kLbRounds = 2;                   // chunks per data wavefront per tile
constexpr int kLbSub = kDataWaves * kChunk;    // 15360 elements per round
constexpr int kTile = kLbSub * kLbRounds;      // 30720 elements per tile
constexpr uint32_t kMaxTiles = 1u << 18;       // power of two >= descriptor words of the largest n
// 128-bit loads per lane of the persistent kernels' 32-bit chunks (2048
// elements per data wavefront, a 30720-element tile). A build with
// SSC_STRESS_TILES defined takes one (3840-element tiles: eight times the
// tiles, claims and look-backs per call) to stress the descriptor protocol in
// the tests; it accepts n up to 2^17 tiles and is no faster.
#ifdef SSC_STRESS_TILES
constexpr int kTileLoads = 1;
#else
constexpr int kTileLoads = 8;
#endif
constexpr int kSelTile = kDataWaves * kWave * kTileLoads * 4;  // elements per compaction tile
// Workgroups of the grid-stride counting kernels: one per compute unit. The
// memory system delivers more with fewer reads waiting (2^28 int32, count of
// the even elements: 1024 / 512 / 256 / 128 workgroups 197 / 176 / 167 /
// 294 us; 162.7 with the next sub-tile's loads issued before the current one
// is counted; the 32-pass radix sort at 2^24 1,184 -> 1,121 us from 512 to 256).
constexpr int kReduceGrid = 256;
constexpr int kSpread = 16;                    // accumulators a counting pass spreads over

static_assert(kLbBlock == (kDataWaves + 1) * kWave, "one control wavefront");
// two words per compaction tile: the wide descriptors of the fp32 scans, and
// the tiles of half the size of the key-value and 64-bit formats
static_assert(kTile % kSelTile == 0, "compaction tiles divide the scan tile");
#ifndef SSC_STRESS_TILES
static_assert(static_cast<int64_t>(kMaxTiles) * kSelTile >= 2LL * 2147483647LL, "kMaxTiles");
#endif

// Scratch header (bytes). Descriptors follow it, one 64-bit word per tile.
constexpr size_t kHeaderBytes = 512;
constexpr size_t kOffClaim = 0;      // uint64 {epoch:32 | next tile:32}
constexpr size_t kOffTimedOut = 8;   // uint32 look-back time-out flag
constexpr size_t kOffDone = 12;      // uint32 workgroups finished (counting passes)
constexpr size_t kOffClaimed = 16;   // uint32 workgroups done claiming (persistent kernels)
constexpr size_t kOffAcc = 64;       // uint32[kSpread] partial counts
constexpr size_t kOffAcc32 = 128;    // uint32[32] per-bit clear counts being summed
constexpr size_t kOffKept32 = 256;   // uint32[32] per-bit clear counts of the current sort

__host__ __device__ constexpr int64_t tiles_for(int64_t n) { return (n + kTile - 1) / kTile; }
// Descriptor words for n elements: two per compaction tile.
__host__ __device__ constexpr int64_t desc_words(int64_t n) { return 2 * ((n + kSelTile - 1) / kSelTile); }

// Four 32-bit lanes moved by one 128-bit global load or store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 32-bit reinterpretation through a scalar value (bit_cast of a vector
// element lvalue is avoided: it does not read the element it names).
template <class T>
__device__ __forceinline__ T from_u32(uint32_t b) {
    return __builtin_bit_cast(T, b);
}
template <class T>
__device__ __forceinline__ uint32_t to_u32(T v) {
    return __builtin_bit_cast(uint32_t, v);
}

struct ScratchView {
    uint64_t *claim;
    uint32_t *timed_out;
    uint32_t *done;
    uint32_t *claimed;
    uint32_t *acc;
    uint32_t *acc32;
    uint32_t *kept32;
    uint64_t *desc;
};

__host__ __device__ inline ScratchView view(void *scratch) {
    char *b = static_cast<char *>(scratch);
    ScratchView v;
    v.claim = reinterpret_cast<uint64_t *>(b + kOffClaim);
    v.timed_out = reinterpret_cast<uint32_t *>(b + kOffTimedOut);
    v.done = reinterpret_cast<uint32_t *>(b + kOffDone);
    v.claimed = reinterpret_cast<uint32_t *>(b + kOffClaimed);
    v.acc = reinterpret_cast<uint32_t *>(b + kOffAcc);
    v.acc32 = reinterpret_cast<uint32_t *>(b + kOffAcc32);
    v.kept32 = reinterpret_cast<uint32_t *>(b + kOffKept32);
    v.desc = reinterpret_cast<uint64_t *>(b + kHeaderBytes);
    return v;
}

// --------------------------------------------------------------- loading ---
// A chunk is the 1024 elements one wavefront owns: element (j, lane, k) is at
// chunk + j*256 + lane*4 + k. `rem` (uniform) is the number of valid
// elements from the chunk's start (>= kChunk: the chunk is full), so validity
// is a 32-bit compare. Addresses are a uniform base (SGPRs) plus one 32-bit
// per-lane byte offset. VEC selects 128-bit accesses (the array is 16-byte
// aligned) or 32-bit ones. Full-chunk 128-bit accesses are nontemporal:
// every byte is touched once, so streaming it past the caches leaves them to
// the descriptors (measured faster on MI355X for GiB-sized arrays).

__device__ __forceinline__ uint32_t chunk_rem(int64_t n, int64_t chunk) {
    const int64_t r = n - chunk;
    return r <= 0 ? 0u : (r >= kChunk ? static_cast<uint32_t>(kChunk) : static_cast<uint32_t>(r));
}

__device__ __forceinline__ bool in_chunk(uint32_t rem, int j, int lane, int k) {
    return static_cast<uint32_t>(j * (kWave * 4) + lane * 4 + k) < rem;
}

template <bool VEC, class T>
__device__ __forceinline__ void load_chunk(const T *__restrict__ in, int64_t chunk, int lane,
                                           uint32_t rem, T (&v)[kLoads][4]) {
    static_assert(sizeof(T) == 4, "32-bit elements");
    const char *base = reinterpret_cast<const char *>(in + chunk);
    const uint32_t lane_off = static_cast<uint32_t>(lane) * 16u;
    if (rem >= static_cast<uint32_t>(kChunk)) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const char *bj = base + j * (kWave * 16);
            if constexpr (VEC) {
                const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(bj + lane_off));
                v[j][0] = from_u32<T>(q[0]);
                v[j][1] = from_u32<T>(q[1]);
                v[j][2] = from_u32<T>(q[2]);
                v[j][3] = from_u32<T>(q[3]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[j][k] = *reinterpret_cast<const T *>(bj + lane_off + 4u * k);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const char *bj = base + j * (kWave * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[j][k] = in_chunk(rem, j, lane, k) ? *reinterpret_cast<const T *>(bj + lane_off + 4u * k)
                                                    : T(0);
        }
    }
}

template <bool VEC, class T>
__device__ __forceinline__ void store_chunk(T *out, int64_t chunk, int lane, uint32_t rem,
                                            const T (&v)[kLoads][4]) {
    char *base = reinterpret_cast<char *>(out + chunk);
    const uint32_t lane_off = static_cast<uint32_t>(lane) * 16u;
    if (rem >= static_cast<uint32_t>(kChunk)) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            char *bj = base + j * (kWave * 16);
            if constexpr (VEC) {
                u32x4 q;
                q[0] = to_u32(v[j][0]);
                q[1] = to_u32(v[j][1]);
                q[2] = to_u32(v[j][2]);
                q[3] = to_u32(v[j][3]);
                __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(bj + lane_off));
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) *reinterpret_cast<T *>(bj + lane_off + 4u * k) = v[j][k];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            char *bj = base + j * (kWave * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (in_chunk(rem, j, lane, k)) *reinterpret_cast<T *>(bj + lane_off + 4u * k) = v[j][k];
        }
    }
}

// Wavefront-local ranks of one chunk. Evaluates the predicate once per valid
// element and records the flags in `mask` at bit (bit0 + j*4 + k).
// lead[j] = flagged elements in earlier loads of the chunk plus those of
// load j in lower lanes; the element's rank inside the chunk is lead[j] +
// (flagged components before k in its lane). Returns the chunk's flag total
// (uniform).
template <int P>
__device__ __forceinline__ uint32_t chunk_ranks(const int32_t (&v)[kLoads][4], int lane,
                                                uint32_t rem, const PredArgs &pr,
                                                uint32_t (&lead)[kLoads], uint64_t &mask,
                                                int bit0) {
    uint32_t running = 0;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        uint32_t below = 0;
        uint32_t total = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool f = in_chunk(rem, j, lane, k) && pred_eval<P>(v[j][k], pr);
            mask |= static_cast<uint64_t>(f) << (bit0 + j * 4 + k);
            const uint64_t m = ballot(f);
            below += mbcnt64(m);
            total += static_cast<uint32_t>(__builtin_popcountll(m));
        }
        lead[j] = running + below;
        running += total;
    }
    return running;
}

__device__ __forceinline__ bool bit(uint64_t mask, int b) { return (mask >> b) & 1u; }

// Chunk totals of a tile live in LDS in (round q, data wavefront d) order,
// s_tot[q * kDataWaves + d]. The last data wavefront to finish scans them
// once (lanes 0..29, one DPP wavefront scan, a fixed order, so the fp32 sums
// are the same for every reader) into s_pre: s_pre[i] = total of chunks
// before chunk i, s_pre[kLbRounds * kDataWaves] = tile aggregate.
constexpr int kChunksPerTile = kLbRounds * kDataWaves;  // 30

template <class Op>
__device__ __forceinline__ typename Op::T scan_chunk_totals(const uint32_t *s_tot, uint32_t *s_pre,
                                                            int lane) {
    using T = typename Op::T;
    const T mine = lane < kChunksPerTile ? Op::from_bits(s_tot[lane]) : Op::zero();
    const T incl = wave_inclusive_scan<Op>(mine);
    const uint32_t up = static_cast<uint32_t>(__shfl_up(static_cast<int>(Op::bits(incl)), 1));
    if (lane < kChunksPerTile) s_pre[lane] = lane == 0 ? Op::bits(Op::zero()) : up;
    const T agg = Op::from_bits(static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(Op::bits(incl)), kChunksPerTile - 1)));
    if (lane == 0) s_pre[kChunksPerTile] = Op::bits(agg);
    return agg;
}

// Offsets for data wavefront w after the barrier that follows the scan:
// chunk_before[q] = total of chunks before (q, w); round_before[q] = total
// of rounds before q; round_before[kLbRounds] = tile aggregate. Uniform.
template <class Op>
__device__ __forceinline__ void tile_prefixes(const uint32_t *s_pre, int w,
                                              typename Op::T (&chunk_before)[kLbRounds],
                                              typename Op::T (&round_before)[kLbRounds + 1]) {
    const int d = w < kDataWaves ? w : 0;
#pragma unroll
    for (int q = 0; q < kLbRounds; ++q) {
        chunk_before[q] = Op::from_bits(uniform(s_pre[q * kDataWaves + d]));
        round_before[q] = Op::from_bits(uniform(s_pre[q * kDataWaves]));
    }
    round_before[kLbRounds] = Op::from_bits(uniform(s_pre[kChunksPerTile]));
}

// Claims the next tile for this workgroup (one thread). Returns
// {epoch:32 | tile:32}. A call makes exactly `claims` claims in all; the one
// that receives the last number resets the counter and advances the epoch
// (every claim of a call therefore carries the same epoch), and clears one
// stale descriptor word: word (epoch mod kMaxTiles) when this call does not
// use it (it uses words 0 .. words_used - 1). Over any kMaxTiles consecutive
// calls every word is thus rewritten or cleared, far within the 2^30-call
// period of the tag, so no stale descriptor can match a later tag.
__device__ __forceinline__ void end_epoch(const ScratchView &sv, uint32_t epoch,
                                          uint32_t words_used, uint32_t capacity) {
    __hip_atomic_store(sv.claim, static_cast<uint64_t>(epoch + 1u) << 32, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t slot = epoch & (kMaxTiles - 1u);
    if (slot >= words_used && slot < capacity)
        __hip_atomic_store(sv.desc + slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t claim_tile(const ScratchView &sv, uint32_t words_used,
                                               uint32_t claims, uint32_t capacity) {
    perturb(blockIdx.x, 8);
    const uint64_t c =
        __hip_atomic_fetch_add(sv.claim, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<uint32_t>(c) == claims - 1)
        end_epoch(sv, static_cast<uint32_t>(c >> 32), words_used, capacity);
    return c;
}

// The persistent kernel's claims: a workgroup claims its first tile, then
// its second and third together (two consecutive numbers, one atomic), then
// one per tile, and stops claiming once it holds a number past the end. Its
// first tile is claimed alone so that first tiles interleave across
// workgroups: were the first three consecutive, each workgroup's first
// look-back would wait for the previous workgroup's third tile, a chain
// through the whole grid. How many
// claims a call makes then depends on timing, so the counter is reset by the
// last workgroup to finish claiming instead: each one counts itself in
// *claimed once, after its last claim has returned, and the one that
// completes the count ends the epoch. Every claim of the call has been
// performed by then, so all carry one epoch.
__device__ __forceinline__ uint64_t claim_tiles(const ScratchView &sv, uint64_t k) {
    perturb(blockIdx.x * 4u + static_cast<uint32_t>(k), 9);
    return __hip_atomic_fetch_add(sv.claim, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void finish_claims(const ScratchView &sv, uint32_t epoch,
                                              uint32_t workgroups, uint32_t words_used,
                                              uint32_t capacity) {
    perturb(blockIdx.x, 10);
    const uint32_t before =
        __hip_atomic_fetch_add(sv.claimed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == workgroups - 1u) {
        __hip_atomic_store(sv.claimed, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        end_epoch(sv, epoch, words_used, capacity);
    }
}

constexpr uint32_t kNoTile = 0xFFFFFFFFu;  // no tile: past the end

// The second and third tiles of a persistent workgroup (control lane 0,
// while the data wavefronts load the first). With at least three tiles per
// workgroup both come from one atomic (one round trip); with fewer they are
// claimed one at a time, so that no workgroup takes two of the last tiles
// while others get none (10^7 int32 scan: 22.4 -> 20.6 us). Returns true when
// the claims reached the end.
__device__ __forceinline__ bool claim_second_third(const ScratchView &sv, uint32_t num_tiles,
                                                   uint32_t *first) {
    uint32_t c1, c2;
    if (num_tiles >= 3u * gridDim.x) {
        c1 = static_cast<uint32_t>(claim_tiles(sv, 2));
        c2 = c1 + 1u;
    } else {
        c1 = static_cast<uint32_t>(claim_tiles(sv, 1));
        c2 = c1 < num_tiles ? static_cast<uint32_t>(claim_tiles(sv, 1)) : kNoTile;
    }
    first[1] = c1;
    first[2] = c2;
    return c2 >= num_tiles;
}

// Arrival of a data wavefront (whole wavefront) after writing its chunk
// totals to LDS. The last of the kDataWaves to arrive scans the totals into
// s_pre and publishes the tile's descriptor at once -- {aggregate, A}, or
// {inclusive, A} for tile 0 -- without waiting for the control wavefront, so a
// slow look-back never delays the successors. (If this store ever lands after
// the control wavefront's later {inclusive} store, successors just walk one
// tile further: both are valid states.)
template <class Op, bool WIDE>
__device__ __forceinline__ void arrive_and_publish(uint32_t *s_arrive, const uint32_t *s_tot,
                                                   uint32_t *s_pre, uint64_t *desc, uint32_t tile,
                                                   uint32_t tag, int lane) {
    perturb(tile * 16u + threadIdx.x / kWave, 11);
    uint32_t before = 0;
    if (lane == 0)
        before = __hip_atomic_fetch_add(s_arrive, 1u, __ATOMIC_ACQ_REL,
                                        __HIP_MEMORY_SCOPE_WORKGROUP);
    if (uniform(before) == kDataWaves - 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const typename Op::T agg = scan_chunk_totals<Op>(s_tot, s_pre, lane);
        const uint32_t st = tile == 0 ? kStatusInclusive : kStatusAggregate;
        if (lane == 0) {
            if constexpr (WIDE)
                publish_wide(desc, tile, tag, st, static_cast<double>(agg));
            else
                publish(desc + tile, tag, st, Op::bits(agg));
        }
    }
}

// ------------------------------------------- buffer-resource chunk access ---
// The persistent compaction kernel reads and writes through buffer
// resources: a resource over `bytes` bytes drops 32-bit lanes past its end
// dword by dword (loads return 0, stores are discarded; a 128-bit load that
// straddles the end keeps its in-range dwords). Partial chunks and
// variable-length runs then need no branches, and every wavefront issues the
// same memory instructions on every tile.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, no swizzle
constexpr int kNT = 2;                  // nontemporal cache policy
constexpr int kStageWords = 2048;       // LDS staging words per data wavefront (8 KiB)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), kRsrcWord3);
}

// The shape of one data wavefront's chunk: L loads per lane of K elements
// each. Element (j, lane, k) is element j*64*K + lane*K + k of the chunk and
// bit j*K + k of the lane's 32-bit flag mask; a tile is one chunk per data
// wavefront.
template <int L, int K>
struct ChunkShape {
    static constexpr int kLoads = L;
    static constexpr int kPer = K;
    static constexpr int kChunk = kWave * L * K;
    static constexpr int kTileElems = kDataWaves * kChunk;
    static_assert(L * K <= 32, "a lane's flags fit one 32-bit mask");
    static_assert(K <= 4, "a load's flag count fits the packed 10-bit fields");
};

template <int C>
__device__ __forceinline__ uint32_t chunk_rem(int64_t n, int64_t chunk) {
    const int64_t r = n - chunk;
    return r <= 0 ? 0u : (r >= C ? static_cast<uint32_t>(C) : static_cast<uint32_t>(r));
}

// Loads L x 4 32-bit elements per lane (rem valid in the chunk) in the
// (j, lane, k) layout; missing elements read as 0. VEC: 128-bit loads, else
// 32-bit ones. Nontemporal: every byte is read once.
template <int L, bool VEC>
__device__ __forceinline__ void load_b32x4(const int32_t *in, int64_t chunk, uint32_t rem,
                                           int lane, int32_t (&v)[L][4]) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(in + chunk, rem * 4u);
    const int lane_off = lane * 16;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        if constexpr (VEC) {
            const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, j * (kWave * 16) + lane_off, 0, kNT);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[j][k] = static_cast<int32_t>(q[k]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[j][k] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(
                    r, j * (kWave * 16) + lane_off + 4 * k, 0, kNT));
        }
    }
}

// Writes run[0 .. len) (LDS words) to out[at .. at + len) with a fixed
// C / 64 + 2 32-bit stores per lane whatever len is: slots past each part
// fall outside its resource and are dropped, so words up to run[C + 63] are
// read (the staging array is padded for that). The run is also cut at n: a
// correct look-back never needs it, a broken one then gives wrong results
// instead of stray writes.
// Cache policy by 128-byte line: the run's partial first and last lines are
// shared with the neighbouring runs and take the default policy, so the L2
// merges them; its whole lines are stored nontemporal. Measured at 2^28:
// 99% kept 386 -> 366 us, partition 564 -> 541 us, 50% kept unchanged
// (all lines nontemporal: slower; all default: the 386 / 564). POL is the
// whole lines' policy: a run the library itself reads next (the radix
// driver's chained partitions) takes the default policy, which keeps it in
// the caches (2^24 keys: 1,265 us against 1,360 us with nontemporal lines).
// HALF: the second half of the C / 64 piece stores only for a run longer
// than half a chunk. Stores past the run's end are dropped by the buffer
// resource, but each still passes through the memory pipeline, and at low
// selectivity nearly all are such. Skipping all of them (one store per
// piece the run has) gained 5.5 us at 1% kept, but the compiler cannot
// count such stores, so its wait for the next chunk's data also waits for
// them (10% kept 215.3 -> 217.5, 25% 225.5 -> 249.4, the headline 266.3 ->
// 282.3). With half always issued the wait covers at most half of them
// (2^28 MOD_LT(100, s): 1% kept 199.7 -> 195.1 us, 5% 216.8 -> 208.8, 10%
// 215.7 -> 207.8, 50% 267.0 -> 264.1; the headline 265.6 -> 265.3; flag
// selection 144.3 -> 141.4, flag-byte compaction 310.8 -> 309.0, int64
// 267.7 -> 266.8). Key-value pairs (266.3 -> 270.9) and partitions (522.6 ->
// 525.2), which write two runs a chunk, issue them all, and so does
// compaction with ranks (464.9 -> 464.7, no gain).
template <int C, int POL = kNT, bool HALF = false>
__device__ __forceinline__ void stream_run(const uint32_t *run, uint32_t *out, uint32_t at,
                                           uint32_t len, int64_t n, int lane) {
    len = uniform(len);
    const int64_t room = n - static_cast<int64_t>(at);
    if (static_cast<int64_t>(len) > room) len = room > 0 ? static_cast<uint32_t>(room) : 0u;
    uint32_t *dst = out + at;
    // words before the run's first 128-byte line boundary
    uint32_t head = static_cast<uint32_t>((128u - (reinterpret_cast<uintptr_t>(dst) & 127u)) & 127u) / 4u;
    head = uniform(head < len ? head : len);
    const uint32_t full = uniform((len - head) / static_cast<uint32_t>(kWave));  // whole 64-word stores
    const uint32_t tail_at = head + full * static_cast<uint32_t>(kWave);
    const int voff = lane * 4;
    __builtin_amdgcn_raw_buffer_store_b32(run[lane], buffer_rsrc(dst, head * 4u), voff, 0, 0);
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(dst + head, full * static_cast<uint32_t>(kWave) * 4u);
    const uint32_t *src = run + head + lane;
    constexpr int kFirst = HALF ? C / kWave / 2 : C / kWave;
#pragma unroll
    for (int i = 0; i < kFirst; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(src[i * kWave], rb, voff + i * (kWave * 4), 0, POL);
    if (kFirst < C / kWave && full > static_cast<uint32_t>(kFirst)) {
#pragma unroll
        for (int i = kFirst; i < C / kWave; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(src[i * kWave], rb, voff + i * (kWave * 4), 0, POL);
    }
    __builtin_amdgcn_raw_buffer_store_b32(run[tail_at + lane],
                                          buffer_rsrc(dst + tail_at, (len - tail_at) * 4u), voff,
                                          0, 0);
}

// Bits of the valid elements (j*64*K + lane*K + k < rem) in the layout of a
// chunk's flag mask.
template <int L, int K>
__device__ __forceinline__ uint32_t valid_mask(int lane, uint32_t rem) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        int left = static_cast<int>(rem) - (j * (kWave * K) + lane * K);
        left = left < 0 ? 0 : (left > K ? K : left);
        m |= ((1u << left) - 1u) << (j * K);
    }
    return m;
}

// Flags of L x 4 32-bit elements as a per-lane mask: bit j*4 + k is the
// predicate of element (j, lane, k), evaluated once; elements past rem are
// not flagged.
//
// The mask is assembled with v_alignbit_b32, which shifts a 64-bit pair
// right and keeps the low word: alignbit(x, m, 1) is m >> 1 with bit 0 of x
// entering at bit 31, so after the 32 elements in order, element e sits at
// bit e. That is one instruction per element for the parity predicates and
// two for NONZERO (min(x, 1) is 1 iff x != 0) and the bit tests, where a
// shift and a mask, or a compare and a select, cost three or four; the fp32
// comparisons enter their 0/1 the same way. MOD_LT
// subtracts the threshold from the residue's fraction (both in [0, 1], so
// the difference is negative, its sign bit set, exactly when the element is
// kept) and shifts that sign bit in from the bottom instead: alignbit(m,
// hi, 31) is m << 1 with bit 31 of hi entering at bit 0, and a bit reversal
// at the end puts element e at bit e.
template <int P, int L>
__device__ __forceinline__ uint32_t mask_b32(const int32_t (&v)[L][4], int lane, uint32_t rem,
                                             const PredArgs &pr) {
    constexpr int kN = L * 4;
    uint32_t mask = 0;
#pragma unroll
    for (int j = 0; j < L; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t u = static_cast<uint32_t>(v[j][k]);
            if constexpr (P == 0 || P == 6) {
                // min(u, 1) written as the instruction (the compiler would
                // turn it into a compare and a select); an fp32 is nonzero
                // iff its bits without the sign are
                const uint32_t b = P == 0 ? u : u << 1;
                uint32_t nz;
                asm("v_min_u32 %0, %1, 1" : "=v"(nz) : "v"(b));
                mask = __builtin_amdgcn_alignbit(nz, mask, 1);
            } else if constexpr (P == 1 || P == 2) {
                mask = __builtin_amdgcn_alignbit(u, mask, 1);
            } else if constexpr (P == 3 || P == 4) {
                mask = __builtin_amdgcn_alignbit(u >> pr.a, mask, 1);
            } else if constexpr (P == 5) {
                const double t = __builtin_fma(static_cast<double>(v[j][k]), pr.inv, pr.half);
                const double d = __builtin_amdgcn_fract(t) - pr.thr;
                const uint32_t hi = static_cast<uint32_t>(__builtin_bit_cast(uint64_t, d) >> 32);
                mask = __builtin_amdgcn_alignbit(mask, hi, 31);
            } else {
                mask = __builtin_amdgcn_alignbit(pred_eval<P>(v[j][k], pr) ? 1u : 0u, mask, 1);
            }
        }
    if constexpr (P == 5) mask = __builtin_bitreverse32(mask);
    if constexpr (kN < 32) mask >>= 32 - kN;  // the first element at bit 0
    if constexpr (P == 2 || P == 4) mask = ~mask & (kN < 32 ? (1u << kN) - 1u : ~0u);
    if (rem < static_cast<uint32_t>(kN * kWave)) mask &= valid_mask<L, 4>(lane, rem);
    return mask;
}

// The chunk's flag total (uniform): a wavefront sum of the lanes' counts.
__device__ __forceinline__ uint32_t chunk_total(uint32_t mask) {
    const uint32_t incl = wave_inclusive_scan<SumU32>(static_cast<uint32_t>(__builtin_popcount(mask)));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
}

// lead[j] = flagged elements of the chunk before element (j, lane, 0): the
// flags of loads before j plus those of load j in lower lanes. A lane's
// per-load counts (0..K each) travel as words of three 10-bit fields, so
// ceil(L / 3) wavefront scans rank all L loads at once (a field's sum over
// 64 lanes is at most 256). Returns the chunk total (uniform).
template <int L, int K>
__device__ __forceinline__ uint32_t chunk_leads(uint32_t mask, uint32_t (&lead)[L]) {
    constexpr int kWords = (L + 2) / 3;
    constexpr uint32_t kLoadBits = (1u << K) - 1u;
    uint32_t word[kWords] = {};
#pragma unroll
    for (int j = 0; j < L; ++j)
        word[j / 3] |= static_cast<uint32_t>(__builtin_popcount((mask >> (j * K)) & kLoadBits))
                       << (10 * (j % 3));
    uint32_t excl[kWords], tot[kWords];
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
        const uint32_t incl = wave_inclusive_scan<SumU32>(word[q]);
        excl[q] = incl - word[q];
        tot[q] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
    }
    uint32_t running = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int sh = 10 * (j % 3);
        lead[j] = running + ((excl[j / 3] >> sh) & 1023u);
        running += (tot[j / 3] >> sh) & 1023u;
    }
    return running;
}

// ranks[i] = seg + (flags before element i in its chunk) for the chunk's rem
// valid elements, written in the load layout of L x 4 32-bit elements.
template <int L, bool VEC>
__device__ __forceinline__ void write_ranks(int32_t *ranks, int64_t chunk, uint32_t rem,
                                            uint32_t seg, uint32_t mask, int lane) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(ranks + chunk, rem * 4u);
    uint32_t lead[L];
    chunk_leads<L, 4>(mask, lead);
#pragma unroll
    for (int j = 0; j < L; ++j) {
        uint32_t x = seg + lead[j];
        uint32_t q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[k] = x;
            x += (mask >> (j * 4 + k)) & 1u;
        }
        if constexpr (VEC) {
            u32x4 v;
            v[0] = q[0];
            v[1] = q[1];
            v[2] = q[2];
            v[3] = q[3];
            __builtin_amdgcn_raw_buffer_store_b128(v, r, j * (kWave * 16) + lane * 16, 0, kNT);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                __builtin_amdgcn_raw_buffer_store_b32(q[k], r, j * (kWave * 16) + lane * 16 + 4 * k,
                                                      0, kNT);
        }
    }
}

// ------------------------------------------------- element formats ---
// What a chunk is made of, for the persistent kernel below: how its loads
// are issued, how an element's flag is taken, and how a survivor is staged
// in the data wavefront's 8 KiB LDS region and written out. The kernel's
// pipeline (claims, arrivals, look-back, barrier) is the same for all.

// Arrays the kernel reads and writes; which ones a format uses is its own.
struct SelArgs {
    const void *in;   // elements (the keys of key-value pairs)
    const void *aux;  // flag bytes (flag formats) or the values of pairs
    void *out;        // compacted elements or keys, or the survivors' positions
    void *out_aux;    // compacted values of pairs
};

// 32-bit elements (int32, or fp32 bits); the predicate reads the element.
// Eight 128-bit loads per lane (kTileLoads): 2048 elements per data wavefront.
template <bool VEC>
struct FmtB32 {
    using Shape = ChunkShape<kTileLoads, 4>;
    static constexpr int L = Shape::kLoads;
    static constexpr bool kVec = VEC;
    static constexpr bool kValues = true;  // element values are loaded
    static constexpr int kSlotWords = 1;  // 32-bit words per staged survivor
    static constexpr bool kFlagFirst = true;  // stage after the next chunk's arrival
    struct Regs {
        int32_t v[L][4];
    };
    __device__ static void load(const SelArgs &a, int64_t chunk, uint32_t rem, int lane, Regs &r) {
        load_b32x4<L, VEC>(static_cast<const int32_t *>(a.in), chunk, rem, lane, r.v);
    }
    template <int P>
    __device__ static uint32_t flags(const Regs &r, int lane, uint32_t rem, const PredArgs &pr) {
        return mask_b32<P, L>(r.v, lane, rem, pr);
    }
    __device__ static void stage(uint32_t *region, uint32_t slot, const Regs &r, int j, int k) {
        region[slot] = static_cast<uint32_t>(r.v[j][k]);
    }
    template <int POL = kNT, bool HALF = false>
    __device__ static void write(const uint32_t *region, const SelArgs &a, uint32_t at,
                                 uint32_t len, int64_t n, int lane) {
        stream_run<Shape::kChunk, POL, HALF>(region, static_cast<uint32_t *>(a.out), at, len, n, lane);
    }
};

// A caller's predicate as one flag byte per element (nonzero keeps), with
// 32-bit elements (VALUES) or without them (selection: positions only).
// The flags of load j arrive as one 32-bit load per lane, four bytes for the
// lane's four elements; the array must be 4-byte aligned, and the word that
// holds the last flag is read whole (never anything past that word).
template <bool VEC, bool VALUES>
struct FmtFlags {
    using Shape = ChunkShape<kTileLoads, 4>;
    static constexpr int L = Shape::kLoads;
    static constexpr bool kVec = VEC;
    static constexpr bool kValues = VALUES;
    static constexpr int kSlotWords = 1;  // 32-bit words per staged survivor
    static constexpr bool kFlagFirst = false;  // stage after the next chunk's arrival
    struct Regs {
        int32_t v[L][4];
        uint32_t f[L];
    };
    __device__ static void load(const SelArgs &a, int64_t chunk, uint32_t rem, int lane, Regs &r) {
        if constexpr (VALUES)
            load_b32x4<L, VEC>(static_cast<const int32_t *>(a.in), chunk, rem, lane, r.v);
        const __amdgpu_buffer_rsrc_t fr =
            buffer_rsrc(static_cast<const uint8_t *>(a.aux) + chunk, (rem + 3u) & ~3u);
#pragma unroll
        for (int j = 0; j < L; ++j)
            r.f[j] = __builtin_amdgcn_raw_buffer_load_b32(fr, j * (kWave * 4) + lane * 4, 0, kNT);
    }
    template <int P>
    __device__ static uint32_t flags(const Regs &r, int lane, uint32_t rem, const PredArgs &) {
        uint32_t mask = 0;
#pragma unroll
        for (int j = 0; j < L; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                mask |= static_cast<uint32_t>(((r.f[j] >> (8 * k)) & 0xFFu) != 0u) << (j * 4 + k);
        if (rem < static_cast<uint32_t>(Shape::kChunk)) mask &= valid_mask<L, 4>(lane, rem);
        return mask;
    }
    __device__ static void stage(uint32_t *region, uint32_t slot, const Regs &r, int j, int k) {
        region[slot] = static_cast<uint32_t>(r.v[j][k]);
    }
    template <int POL = kNT>
    __device__ static void write(const uint32_t *region, const SelArgs &a, uint32_t at,
                                 uint32_t len, int64_t n, int lane) {
        stream_run<Shape::kChunk, POL, true>(region, static_cast<uint32_t *>(a.out), at, len, n,
                                             lane);
    }
};

// Key-value pairs: 32-bit keys (the predicate reads them) and 32-bit values
// that travel with them. Four 128-bit loads per lane of each array (half of
// kTileLoads, rounded up): 1024 pairs per data wavefront, keys staged in the
// first half of the region and values in the second.
template <bool VEC>
struct FmtPairs {
    using Shape = ChunkShape<(kTileLoads + 1) / 2, 4>;
    static constexpr int L = Shape::kLoads;
    static constexpr bool kVec = VEC;
    static constexpr bool kValues = true;
    static constexpr int kSlotWords = 1;  // 32-bit words per staged survivor
    static constexpr bool kFlagFirst = true;  // stage after the next chunk's arrival
    struct Regs {
        int32_t k[L][4];
        int32_t v[L][4];
    };
    __device__ static void load(const SelArgs &a, int64_t chunk, uint32_t rem, int lane, Regs &r) {
        load_b32x4<L, VEC>(static_cast<const int32_t *>(a.in), chunk, rem, lane, r.k);
        load_b32x4<L, VEC>(static_cast<const int32_t *>(a.aux), chunk, rem, lane, r.v);
    }
    template <int P>
    __device__ static uint32_t flags(const Regs &r, int lane, uint32_t rem, const PredArgs &pr) {
        return mask_b32<P, L>(r.k, lane, rem, pr);
    }
    __device__ static void stage(uint32_t *region, uint32_t slot, const Regs &r, int j, int k) {
        region[slot] = static_cast<uint32_t>(r.k[j][k]);
        region[Shape::kChunk + slot] = static_cast<uint32_t>(r.v[j][k]);
    }
    template <int POL = kNT>
    __device__ static void write(const uint32_t *region, const SelArgs &a, uint32_t at,
                                 uint32_t len, int64_t n, int lane) {
        stream_run<Shape::kChunk, POL>(region, static_cast<uint32_t *>(a.out), at, len, n, lane);
        stream_run<Shape::kChunk, POL>(region + Shape::kChunk, static_cast<uint32_t *>(a.out_aux),
                                       at, len, n, lane);
    }
};

// The predicates on a 64-bit element's two's-complement bits: nonzero, odd,
// even, bit pa (0..63) set or clear.
template <int P>
__device__ __forceinline__ bool pred_eval64(uint64_t u, const PredArgs &pr) {
    if constexpr (P == 0) {
        return u != 0u;
    } else if constexpr (P == 1) {
        return (u & 1u) != 0u;
    } else if constexpr (P == 2) {
        return (u & 1u) == 0u;
    } else if constexpr (P == 3) {
        return ((u >> pr.a) & 1u) != 0u;
    } else {
        static_assert(P == 4, "64-bit predicates: nonzero, odd, even, bit set, bit clear");
        return ((u >> pr.a) & 1u) == 0u;
    }
}

// 64-bit elements: eight 128-bit loads per lane (kTileLoads) of two elements
// each, 1024 elements per data wavefront (8-byte aligned arrays take 64-bit
// loads).
template <bool VEC>
struct FmtB64 {
    using Shape = ChunkShape<kTileLoads, 2>;
    static constexpr int L = Shape::kLoads;
    static constexpr bool kVec = VEC;
    static constexpr bool kValues = true;
    static constexpr int kSlotWords = 2;  // 32-bit words per staged survivor
    static constexpr bool kFlagFirst = false;  // stage after the next chunk's arrival
    struct Regs {
        uint64_t v[L][2];
    };
    __device__ static void load(const SelArgs &a, int64_t chunk, uint32_t rem, int lane, Regs &r) {
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc(static_cast<const uint64_t *>(a.in) + chunk, rem * 8u);
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int off = j * (kWave * 16) + lane * 16;
            if constexpr (VEC) {
                const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
                r.v[j][0] = static_cast<uint64_t>(q[0]) | (static_cast<uint64_t>(q[1]) << 32);
                r.v[j][1] = static_cast<uint64_t>(q[2]) | (static_cast<uint64_t>(q[3]) << 32);
            } else {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const u32x2 d = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8 * k, 0, kNT);
                    r.v[j][k] = static_cast<uint64_t>(d[0]) | (static_cast<uint64_t>(d[1]) << 32);
                }
            }
        }
    }
    template <int P>
    __device__ static uint32_t flags(const Regs &r, int lane, uint32_t rem, const PredArgs &pr) {
        uint32_t mask = 0;
#pragma unroll
        for (int j = 0; j < L; ++j)
#pragma unroll
            for (int k = 0; k < 2; ++k)
                mask |= static_cast<uint32_t>(pred_eval64<P>(r.v[j][k], pr)) << (j * 2 + k);
        if (rem < static_cast<uint32_t>(Shape::kChunk)) mask &= valid_mask<L, 2>(lane, rem);
        return mask;
    }
    __device__ static void stage(uint32_t *region, uint32_t slot, const Regs &r, int j, int k) {
        reinterpret_cast<uint64_t *>(region)[slot] = r.v[j][k];
    }
    template <int POL = kNT>
    __device__ static void write(const uint32_t *region, const SelArgs &a, uint32_t at,
                                 uint32_t len, int64_t n, int lane) {
        // A run of 64-bit elements is a run of twice as many 32-bit words, and
        // goes out as one (256 bytes per store instruction). 64-bit stores
        // (512 bytes per instruction) measured slower at 2^27 int64: 272.9 ->
        // 266.7 us with 50% kept, 374.7 -> 366.6 us with all kept. 2 * at
        // stays below 2^32 for every n the calls accept.
        stream_run<2 * Shape::kChunk, POL, true>(region, static_cast<uint32_t *>(a.out), 2u * at,
                                           2u * len, 2 * n, lane);
    }
};

// ===================================================== compaction kernel ---
// Persistent form: one 1024-thread workgroup per compute unit (its LDS and
// 128 VGPRs per lane fill the unit) loops over tiles whose numbers come from
// the atomic counter, claimed three ahead (the second and third with one
// atomic, while the first is loading). A tile is one chunk for each of the
// 15 data wavefronts (for 32-bit elements 2048 of them, eight 128-bit loads
// per lane: 30720 per tile); the 16th is the control wavefront.
//
// Per tile, a data wavefront holds two chunks in registers: the current
// tile's, already flagged and ranked, and the next tile's, in flight. It
//   1. stages the current chunk's survivors at their rank in its own LDS
//      region (for a partition the rejected ones after them);
//   2. issues the loads of the tile after next into the registers that just
//      freed up (with a third register set, before step 1: see three_sets);
//   3. flags the next tile's chunk (waiting only for those loads), writes
//      its total to LDS and arrives; the last of the 15 to arrive scans the
//      totals and publishes the next tile's {aggregate} at once (with three
//      sets the 32-bit and key-value formats take this step before step 1:
//      see kFlagFirst);
//   4. waits at the tile's one workgroup barrier for the base (the survivors
//      of all earlier tiles) that the control wavefront found;
//   5. writes its region out to out[base + chunk prefix].
// The control wavefront claims a tile, walks the look-back for the current
// tile's base, passes the barrier and publishes {inclusive}. So every tile's
// aggregate goes out before its workgroup waits on anything, and the next
// two tiles' loads are in flight during both the look-back wait and the
// write-out.
//
// Memory instructions per wavefront and tile are fixed (loads and stores go
// through buffer resources that drop what lies past a chunk's or a run's
// end), so the compiler's waits name exact counts: step 3 waits for the
// next chunk's loads and never for the loads issued in step 2. The lane
// number is made opaque once per tile so that address arithmetic stays in
// the loop, folded into instruction offsets, instead of being hoisted into
// registers held across it.
//
// Forward progress: only running workgroups hold tiles (every tile number
// comes from a claim), a workgroup processes its claims in increasing order,
// and it stops claiming after its first number past the end. The lowest
// unfinished tile is the current tile of the workgroup that claimed it (any
// earlier claim of that workgroup is lower and finished), and its look-back
// needs only lower, finished tiles; so the kernel finishes whichever of its
// workgroups are resident at once.
// KIND: compaction (survivors' values), compaction that also writes the
// ranks, stable partition, or selection (survivors' indices).
// kPartitionCached is a partition whose output the library reads with its
// next launch (the radix driver's chained splits): its runs are stored with
// the default cache policy throughout.
enum { kCompact = 0, kCompactRanks = 1, kPartition = 2, kSelectIndex = 3, kPartitionCached = 4 };

// Register sets per data wavefront. With two, the loads of the tile after next
// reuse the current chunk's registers, so they leave only once that chunk is
// staged; with three they leave before the staging. Which one a kernel takes
// is measured (2^28 elements, microseconds per launch, two sets -> three):
//   three: odd 50% kept 286.4 -> 267.1, odd 1% 210.4 -> 201.7, odd
//     selection 284.2 -> 267.0, key-value pairs 284.8 -> 268.4, int64
//     279.6 -> 273.1, flag-byte compaction 327.2 -> 310.2;
//   two: ranks 463 -> 476, partitions 537 -> 540, the radix driver's
//     chained splits (2^24 keys, 1,176 -> 1,210 a sort);
//   MOD_LT(100, s) with the residue read off a fraction (four fp64
//     operations per element): 1% kept 211.9 -> 206.7, 10% 229.6 -> 219.1,
//     50% 268.3 -> 268.0. (With the earlier seven-operation residue, three
//     sets lost below a quarter kept: 1% 216 -> 226.)
template <class F, int P, int KIND>
constexpr bool three_sets() {
    return (KIND == kCompact || KIND == kSelectIndex) && F::kValues;
}
// The look-back with three sets (MOD_LT aside) goes straight to its window and
// polls at s_sleep 32; with two it first waits on its predecessor and polls
// at s_sleep 16 (each measured best for its pipeline; MOD_LT with three sets
// polls as with two: 50% kept 273.5 -> 269.5, 1% 229.4 -> 225.9).
// Forms of the persistent compaction kernel (FORM in select_kernel).
constexpr int kFormDefault = 0;
constexpr int kFormDense = 1;

template <bool THREE>
constexpr int sel_poll_sleep() {
    return THREE ? 32 : 16;
}

// F is the element format (what a chunk holds and how survivors are staged
// and written); partition and ranks are defined for 32-bit elements.
template <class F, int P, int KIND, int FORM = kFormDefault>
__global__ __launch_bounds__(kLbBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void select_kernel(
    SelArgs a, int64_t n, PredArgs pr, void *scratch, uint32_t num_tiles, uint32_t capacity,
    int32_t *__restrict__ count, int32_t *__restrict__ ranks,
    const int32_t *__restrict__ kept_total) {
    using S = typename F::Shape;
    static_assert(KIND == kCompact || KIND == kSelectIndex || __is_same(F, FmtB32<F::kVec>),
                  "partition and ranks take 32-bit elements");
    constexpr bool kPart = KIND == kPartition || KIND == kPartitionCached;
    constexpr int kRunPol = KIND == kPartitionCached ? 0 : kNT;  // whole lines of the runs
    // one staging region per data wavefront, plus two of padding for run reads
    // (a partition's second run starts inside its region)
    __shared__ __attribute__((aligned(16))) uint32_t s_stage[kDataWaves + 2][kStageWords];
    __shared__ uint32_t s_tot[kDataWaves];
    __shared__ uint32_t s_pre[3][kDataWaves + 1];  // chunk prefixes + aggregate, by tile mod 3
    __shared__ uint32_t s_base[2], s_next[2];      // by tile parity
    __shared__ uint32_t s_first[3], s_epoch, s_arrive;

    constexpr bool kThree = three_sets<F, P, KIND>();
    // With three sets, the 32-bit and key-value formats flag the next chunk
    // and arrive before staging the current one, so the next tile's
    // aggregate goes out as soon as its data has landed and the staging
    // fills the wait at the barrier (2^28 MOD_LT(100, 1): 200.1 -> 197.9 us,
    // key-value pairs 263.3 -> 261.6; MOD_LT(100, 99) 349.1 -> 349.8, int64
    // 261.4 -> 262.0, and flag-byte compaction, at the register cap, 309 ->
    // 361, keep the other order).
    constexpr bool kFlagFirst = kThree && F::kFlagFirst;
    // The form, chosen on the host for MOD_LT(m, s) from the fraction s/m it
    // keeps of uniform input. Dense (4s >= 3m): the look-back goes straight
    // to its window and the tile after next's loads leave after the next
    // chunk's arrival. At 99% kept the write stream dominates and both help
    // (365.6 -> 359.3 us at 2^28); at 50% the late loads cost 11.5 us, and
    // below about half kept the predecessor poll pays off. Either form is
    // correct for any input; only the speed depends on the fraction kept.
    constexpr bool kDense = FORM == kFormDense && kThree && kFlagFirst;
    // one 32-bit run a chunk: its second half of stores only when needed
    constexpr bool kHalf = (KIND == kCompact || KIND == kSelectIndex) && __is_same(F, FmtB32<F::kVec>);
    constexpr bool kLbFast = kThree && (P != 5 || kDense);  // look-back without the predecessor poll
    const ScratchView sv = view(scratch);
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    if (threadIdx.x == 0) {
        const uint64_t c = claim_tiles(sv, 1);
        s_first[0] = static_cast<uint32_t>(c);
        s_epoch = static_cast<uint32_t>(c >> 32);
        s_arrive = 0;
    }
    __syncthreads();  // B0: the first tile
    uint32_t tile = uniform(s_first[0]);
    const uint32_t epoch = uniform(s_epoch);
    const uint32_t tag = epoch & kTagMask;
    if (tile >= num_tiles) {  // nothing left for this workgroup
        if (w == kCtrlWave && lane == 0) finish_claims(sv, epoch, gridDim.x, num_tiles, capacity);
        return;
    }
    bool last_claim = false;  // control lane 0: the claims just made reached the end
    if (w == kCtrlWave && lane == 0) last_claim = claim_second_third(sv, num_tiles, s_first);
    uint32_t par = 0;  // tile parity within the workgroup: s_base, s_next
    uint32_t tri = 0;  // tile number within the workgroup mod 3: s_pre

    if (w == kCtrlWave) {
        __syncthreads();  // B0b: the second and third tiles
        uint32_t nxt = uniform(s_first[1]);
        uint32_t nxt2 = uniform(s_first[2]);
        __syncthreads();  // B0': the first tile's arrivals are in
        while (true) {
            uint32_t nxt3 = kNoTile;
            if (lane == 0 && nxt2 < num_tiles) {
                nxt3 = static_cast<uint32_t>(claim_tiles(sv, 1));
                last_claim = nxt3 >= num_tiles;
            }
            uint32_t prefix = 0;
            if (tile != 0)
                prefix = look_back<SumU32, sel_poll_sleep<kLbFast>(), !kLbFast>(sv.desc, tile, tag,
                                                                                sv.timed_out);
            if (lane == 0) {
                s_base[par] = prefix;
                s_next[par] = nxt3;
            }
            __syncthreads();  // B1
            const uint32_t agg = uniform(s_pre[tri][kDataWaves]);
            if (lane == 0) {
                if (tile != 0) publish(sv.desc + tile, tag, kStatusInclusive, prefix + agg);
                if (!kPart && tile == num_tiles - 1)
                    *count = static_cast<int32_t>(prefix + agg);
                // after the barrier: the count's atomic round trip stays off
                // the path to this tile's base
                if (last_claim) finish_claims(sv, epoch, gridDim.x, num_tiles, capacity);
                last_claim = false;
            }
            if (nxt >= num_tiles) return;
            tile = nxt;
            nxt = nxt2;
            nxt2 = uniform(nxt3);
            par ^= 1u;
            tri = tri == 2u ? 0u : tri + 1u;
        }
    }

    const uint32_t kept = kPart ? static_cast<uint32_t>(*kept_total) : 0u;
    typename F::Regs va, vb, vc;  // vc: the third set (kThree)
    uint32_t fm_cur = 0, fm_nxt = 0;  // flags of the current / next chunk
    uint32_t a_cur = 0, a_nxt = 0;    // their totals
    uint32_t rem_cur = 0, rem_nxt = 0;
    const auto chunk_of = [&](uint32_t t) {
        return static_cast<int64_t>(t) * S::kTileElems + static_cast<int64_t>(w) * S::kChunk;
    };
    // a tile past the end has no valid elements: its loads touch nothing
    const auto rem_of = [&](uint32_t t) {
        return t < num_tiles ? chunk_rem<S::kChunk>(n, chunk_of(t)) : 0u;
    };

    // Flags of chunk V (tile T, R valid) into FM and A, then the arrival: the
    // last data wavefront to arrive scans the 15 totals into s_pre[TRI] and
    // publishes T's {aggregate} ({inclusive} for tile 0).
#define SSC_FLAG_AND_ARRIVE(V, T, R, FM, A, TRI, LN)                                          \
    {                                                                                         \
        FM = F::template flags<P>(V, LN, R, pr);                                              \
        A = chunk_total(FM);                                                                  \
        if (LN == 0) s_tot[w] = A;                                                            \
        perturb((T) * 16u + w, 11);                                                           \
        uint32_t before_ = 0;                                                                 \
        if (LN == 0)                                                                          \
            before_ = __hip_atomic_fetch_add(&s_arrive, 1u, __ATOMIC_ACQ_REL,                 \
                                             __HIP_MEMORY_SCOPE_WORKGROUP);                   \
        if (uniform(before_) == kDataWaves - 1) {                                             \
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");                            \
            const uint32_t mine_ = LN < kDataWaves ? s_tot[LN] : 0u;                          \
            const uint32_t incl_ = wave_inclusive_scan<SumU32>(mine_);                        \
            if (LN < kDataWaves) s_pre[TRI][LN] = incl_ - mine_;                              \
            const uint32_t agg_ = static_cast<uint32_t>(                                      \
                __builtin_amdgcn_readlane(static_cast<int>(incl_), kDataWaves - 1));          \
            if (LN == 0) {                                                                    \
                s_arrive = 0;                                                                 \
                s_pre[TRI][kDataWaves] = agg_;                                                \
                if ((T) < num_tiles)                                                          \
                    publish(sv.desc + (T), tag, (T) == 0 ? kStatusInclusive : kStatusAggregate, \
                            agg_);                                                            \
            }                                                                                 \
        }                                                                                     \
    }

    // One tile (steps 1-5 above) with CUR holding the current chunk, NX the
    // next one in flight and, with three sets, FREE the registers of the chunk
    // staged one tile ago; the loop below rotates the register sets.
    // Stages chunk CUR's survivors at their rank in this wavefront's LDS region
    // (a partition: every element, the rejected ones after the survivors).
#define SSC_STAGE(CUR)                                                                        \
    {                                                                                         \
            /* a partition gives every element a slot of its own, no branches:   */            \
            /* survivors at their rank, the others after all survivors at a_cur + */            \
            /* (index - rank), elements past rem included (they land past the     */            \
            /* runs); compaction and selection stage the survivors only           */            \
            uint32_t lead[S::kLoads];                                                         \
            chunk_leads<S::kLoads, S::kPer>(fm_cur, lead);                                    \
            /* (a selection stages each element's index instead of its value)    */            \
            const int32_t first = static_cast<int32_t>(chunk_of(tile)) + ln * S::kPer;        \
            _Pragma("unroll") for (int j = 0; j < S::kLoads; ++j) {                           \
                if constexpr (kPart) {                                                        \
                    uint32_t r = lead[j];                                                     \
                    const uint32_t rej =                                                      \
                        a_cur + static_cast<uint32_t>(j * (kWave * S::kPer) + ln * S::kPer);  \
                    _Pragma("unroll") for (int k = 0; k < S::kPer; ++k) {                     \
                        const uint32_t f = (fm_cur >> (j * S::kPer + k)) & 1u;                \
                        F::stage(s_stage[w], f ? r : rej + k - r, CUR, j, k);                 \
                        r += f;                                                               \
                    }                                                                         \
                } else {                                                                      \
                    /* a running LDS pointer that each element's flag advances; */           \
                    /* the flag is opaque so that the test reuses the extracted */           \
                    /* bit (else it is taken from the mask a second time)       */           \
                    /* (a selection stages one 32-bit position per survivor)    */           \
                    constexpr int kSlot = KIND == kSelectIndex ? 1 : F::kSlotWords;           \
                    uint32_t *p = s_stage[w] + lead[j] * kSlot;                               \
                    _Pragma("unroll") for (int k = 0; k < S::kPer; ++k) {                     \
                        uint32_t f = __builtin_amdgcn_ubfe(fm_cur, j * S::kPer + k, 1);       \
                        asm volatile("" : "+v"(f));                                           \
                        if (f) {                                                              \
                            if constexpr (KIND == kSelectIndex)                               \
                                *p = static_cast<uint32_t>(first + (j * (kWave * S::kPer) + k)); \
                            else                                                              \
                                F::stage(p, 0, CUR, j, k);                                    \
                        }                                                                     \
                        p += f * kSlot;                                                       \
                    }                                                                         \
                }                                                                             \
            }                                                                                 \
    }

#define SSC_TILE(CUR, NX, FREE)                                                               \
    {                                                                                         \
        int ln = lane;                                                                        \
        asm volatile("" : "+v"(ln));                                                          \
        if constexpr (kThree && !kDense) F::load(a, chunk_of(nxt2), rem_of(nxt2), ln, FREE);  \
        if constexpr (!kFlagFirst) SSC_STAGE(CUR)                                             \
        if constexpr (!kThree) F::load(a, chunk_of(nxt2), rem_of(nxt2), ln, CUR);             \
        const uint32_t tri_n = tri == 2u ? 0u : tri + 1u;                                     \
        rem_nxt = rem_of(nxt);                                                                \
        SSC_FLAG_AND_ARRIVE(NX, nxt, rem_nxt, fm_nxt, a_nxt, tri_n, ln)                       \
        if constexpr (kDense) F::load(a, chunk_of(nxt2), rem_of(nxt2), ln, FREE);             \
        if constexpr (kFlagFirst) SSC_STAGE(CUR)                                              \
        __syncthreads(); /* B1: this tile's base is known */                                  \
        /* the ranks' leads come from fm_cur after the barrier: computed before  */           \
        /* it, they stayed live across the next chunk's flags and the kernel     */           \
        /* spilled (MOD_LT 24 dwords per lane; 485 -> 465 us at 2^28)            */           \
        if constexpr (KIND == kCompactRanks) asm volatile("" : "+v"(fm_cur));                 \
        const uint32_t base = uniform(s_base[par]);                                           \
        const uint32_t nxt3 = uniform(s_next[par]);                                           \
        const int64_t chunk_now = chunk_of(tile);                                             \
        const uint32_t seg = base + uniform(s_pre[tri][w]); /* kept before this chunk */      \
        if constexpr (KIND == kSelectIndex)                                                   \
            stream_run<S::kChunk, kNT, kHalf>(s_stage[w], static_cast<uint32_t *>(a.out), seg,  \
                                              a_cur, n, ln);                                  \
        else if constexpr (kHalf)                                                             \
            F::template write<kRunPol, true>(s_stage[w], a, seg, a_cur, n, ln);               \
        else                                                                                  \
            F::template write<kRunPol>(s_stage[w], a, seg, a_cur, n, ln);                     \
        if constexpr (kPart) {                                                                \
            /* rejected before this chunk = elements before it - kept before it */            \
            const uint32_t rej = static_cast<uint32_t>(chunk_now) - seg;                      \
            F::template write<kRunPol>(s_stage[w] + a_cur, a, kept + rej, rem_cur - a_cur, n, ln); \
        }                                                                                     \
        if constexpr (KIND == kCompactRanks)                                                  \
            write_ranks<S::kLoads, F::kVec>(ranks, chunk_now, rem_cur, seg, fm_cur, ln);      \
        /* advance on every path; the caller leaves once tile is past the end */              \
        tile = nxt;                                                                           \
        nxt = nxt2;                                                                           \
        nxt2 = nxt3;                                                                          \
        par ^= 1u;                                                                            \
        tri = tri_n;                                                                          \
        fm_cur = fm_nxt;                                                                      \
        a_cur = a_nxt;                                                                        \
        rem_cur = rem_nxt;                                                                    \
    }

    rem_cur = rem_of(tile);
    F::load(a, chunk_of(tile), rem_cur, lane, va);
    __syncthreads();  // B0b: the second and third tiles
    uint32_t nxt = uniform(s_first[1]);
    uint32_t nxt2 = uniform(s_first[2]);
    F::load(a, chunk_of(nxt), rem_of(nxt), lane, vb);
    SSC_FLAG_AND_ARRIVE(va, tile, rem_cur, fm_cur, a_cur, tri, lane)
    // B0': without it a fast wavefront could arrive for the next tile
    // before a slow one has arrived for this one
    __syncthreads();
    if constexpr (kThree) {
        while (true) {
            SSC_TILE(va, vb, vc)
            if (tile >= num_tiles) break;
            SSC_TILE(vb, vc, va)
            if (tile >= num_tiles) break;
            SSC_TILE(vc, va, vb)
            if (tile >= num_tiles) break;
        }
    } else {
        while (true) {
            SSC_TILE(va, vb, va)
            if (tile >= num_tiles) break;
            SSC_TILE(vb, va, vb)
            if (tile >= num_tiles) break;
        }
    }
#undef SSC_TILE
#undef SSC_STAGE
#undef SSC_FLAG_AND_ARRIVE
}

// ================================================== flag-byte selection ---
// Selection by flag bytes (idx[k] = position of the k-th nonzero flag) with
// tiles twice the compaction kernel's. A flag is one byte, so a 30720-flag
// tile is too little data to hide the look-back and the barrier each tile
// costs. Here each data lane loads four 128-bit words of flags (4096 per data
// wavefront, 61,440 per tile) and turns them into two 32-bit masks as soon
// as they land. The bytes are then dead, so two raw register sets keep two
// tiles of loads in flight. After the tile's barrier a wavefront writes its
// survivors' positions in two rounds of two loads (2048 flags each), every
// round staged in its 8 KiB LDS region and streamed out as one run. The
// claims, arrivals, look-back and control wavefront are the compaction
// kernel's. The flag array must be 16-byte aligned.
//
// Tile size, 2^28 flags, 50% kept (us per launch): 30,720 flags 158.4,
// 61,440 143.7, 92,160 151.3, 122,880 155.4. Larger tiles cost fewer
// look-backs, but each tile's look-back then waits longer on predecessors
// whose workgroups have fallen behind: at 122,880 flags a tile took 10-20 us,
// and in one tile of six the look-back polled its predecessor more than six
// times (90th percentile 11.5 us).
constexpr int kFlagLoads = kTileLoads == 8 ? 4 : 2;              // 128-bit loads per lane
constexpr int kFlagMasks = kFlagLoads / 2;                        // 32-bit masks per lane
constexpr int kFlagChunk = kWave * 16 * kFlagLoads;               // 4096 flags per data wavefront
constexpr int64_t kFlagTile = static_cast<int64_t>(kDataWaves) * kFlagChunk;  // 61,440
static_assert(kFlagTile >= kSelTile, "at most one descriptor per compaction tile");

// The nonzero bytes of a 32-bit word as a 4-bit mask (bit i = byte i). Bit 7
// of each byte of ((w & 0x7F7F7F7F) + 0x7F7F7F7F) | w is set iff that byte
// is nonzero (no carry leaves a byte); multiplying the four bits, moved to
// bits 0, 8, 16, 24, by 2^24 + 2^17 + 2^10 + 2^3 puts byte i's bit at
// bit 24 + i, with no other product term at or above bit 24 below bit 32.
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
    const uint32_t hi = (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
    return ((hi >> 7) * 0x01020408u) >> 24;
}

__global__ __launch_bounds__(kLbBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void select_flags_kernel(
    const uint8_t *__restrict__ flags, int32_t *__restrict__ idx, int64_t n, void *scratch,
    uint32_t num_tiles, uint32_t capacity, int32_t *__restrict__ count) {
    // one staging region per data wavefront, plus one of padding for run reads
    __shared__ __attribute__((aligned(16))) uint32_t s_stage[kDataWaves + 1][kStageWords];
    __shared__ uint32_t s_tot[kDataWaves];
    __shared__ uint32_t s_pre[3][kDataWaves + 1];  // chunk prefixes + aggregate, by tile mod 3
    __shared__ uint32_t s_base[2], s_next[2];      // by tile parity
    __shared__ uint32_t s_first[3], s_epoch, s_arrive;
    static_assert(kWave * 16 * 2 == kStageWords, "a round of two loads fills one staging region");

    const ScratchView sv = view(scratch);
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    if (threadIdx.x == 0) {
        const uint64_t c = claim_tiles(sv, 1);
        s_first[0] = static_cast<uint32_t>(c);
        s_epoch = static_cast<uint32_t>(c >> 32);
        s_arrive = 0;
    }
    __syncthreads();  // B0: the first tile
    uint32_t tile = uniform(s_first[0]);
    const uint32_t epoch = uniform(s_epoch);
    const uint32_t tag = epoch & kTagMask;
    if (tile >= num_tiles) {
        if (w == kCtrlWave && lane == 0) finish_claims(sv, epoch, gridDim.x, num_tiles, capacity);
        return;
    }
    bool last_claim = false;
    if (w == kCtrlWave && lane == 0) last_claim = claim_second_third(sv, num_tiles, s_first);
    uint32_t par = 0;
    uint32_t tri = 0;

    if (w == kCtrlWave) {
        __syncthreads();  // B0b: the second and third tiles
        uint32_t nxt = uniform(s_first[1]);
        uint32_t nxt2 = uniform(s_first[2]);
        __syncthreads();  // B0': the first tile's arrivals are in
        while (true) {
            uint32_t nxt3 = kNoTile;
            if (lane == 0 && nxt2 < num_tiles) {
                nxt3 = static_cast<uint32_t>(claim_tiles(sv, 1));
                last_claim = nxt3 >= num_tiles;
            }
            uint32_t prefix = 0;
            if (tile != 0) prefix = look_back<SumU32, 16, true>(sv.desc, tile, tag, sv.timed_out);
            if (lane == 0) {
                s_base[par] = prefix;
                s_next[par] = nxt3;
            }
            __syncthreads();  // B1
            const uint32_t agg = uniform(s_pre[tri][kDataWaves]);
            if (lane == 0) {
                // {inclusive} at least one barrier after this tile's {aggregate}
                if (tile != 0) publish(sv.desc + tile, tag, kStatusInclusive, prefix + agg);
                if (tile == num_tiles - 1) *count = static_cast<int32_t>(prefix + agg);
                if (last_claim) finish_claims(sv, epoch, gridDim.x, num_tiles, capacity);
                last_claim = false;
            }
            if (nxt >= num_tiles) return;
            tile = nxt;
            nxt = nxt2;
            nxt2 = uniform(nxt3);
            par ^= 1u;
            tri = tri == 2u ? 0u : tri + 1u;
        }
    }

    const auto chunk_of = [&](uint32_t t) {
        return static_cast<int64_t>(t) * kFlagTile + static_cast<int64_t>(w) * kFlagChunk;
    };
    const auto rem_of = [&](uint32_t t) {
        return t < num_tiles ? chunk_rem<kFlagChunk>(n, chunk_of(t)) : 0u;
    };
    // Four 128-bit words of flags per lane: byte b of load j is flag
    // chunk + j*1024 + lane*16 + b. The resource covers the valid flags
    // rounded up to whole dwords (the dword holding the last flag is read
    // whole: 4-byte aligned, it never crosses a page); the rest read as 0.
    const auto load = [&](uint32_t t, int ln, u32x4(&v)[kFlagLoads]) {
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(flags + chunk_of(t), (rem_of(t) + 3u) & ~3u);
#pragma unroll
        for (int j = 0; j < kFlagLoads; ++j)
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, j * (kWave * 16) + ln * 16, 0, kNT);
    };
    // m[q] = the flags of loads 2q (bits 0-15) and 2q+1 (bits 16-31), those
    // past rem cleared. Returns the chunk's total.
    const auto masks = [&](const u32x4(&v)[kFlagLoads], uint32_t rem, int ln, uint32_t(&m)[kFlagMasks]) {
        uint32_t tot = 0;
#pragma unroll
        for (int q = 0; q < kFlagMasks; ++q) {
            uint32_t x = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int k = 0; k < 4; ++k) x |= nonzero_bytes(v[2 * q + h][k]) << (16 * h + 4 * k);
            if (rem < static_cast<uint32_t>(kFlagChunk)) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int32_t lim = static_cast<int32_t>(rem) - ((2 * q + h) * (kWave * 16) + ln * 16);
                    const uint32_t keep =
                        lim >= 16 ? 0xFFFFu : (lim <= 0 ? 0u : (1u << static_cast<uint32_t>(lim)) - 1u);
                    x &= ~(0xFFFFu << (16 * h)) | (keep << (16 * h));
                }
            }
            m[q] = x;
            tot += static_cast<uint32_t>(__builtin_popcount(x));
        }
        return tot;
    };
    // The last data wavefront to arrive scans the 15 totals into s_pre[TRI]
    // and publishes tile T's {aggregate} ({inclusive} for tile 0).
    const auto arrive = [&](uint32_t lane_tot, uint32_t t, uint32_t tri_, int ln) {
        const uint32_t a = static_cast<uint32_t>(
            __builtin_amdgcn_readlane(static_cast<int>(wave_inclusive_scan<SumU32>(lane_tot)), kWave - 1));
        if (ln == 0) s_tot[w] = a;
        perturb(t * 16u + w, 11);
        uint32_t before = 0;
        if (ln == 0)
            before = __hip_atomic_fetch_add(&s_arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (uniform(before) == kDataWaves - 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            const uint32_t mine = ln < kDataWaves ? s_tot[ln] : 0u;
            const uint32_t incl = wave_inclusive_scan<SumU32>(mine);
            if (ln < kDataWaves) s_pre[tri_][ln] = incl - mine;
            const uint32_t agg =
                static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kDataWaves - 1));
            if (ln == 0) {
                s_arrive = 0;
                s_pre[tri_][kDataWaves] = agg;
                if (t < num_tiles) publish(sv.desc + t, tag, t == 0 ? kStatusInclusive : kStatusAggregate, agg);
            }
        }
    };
    // The survivors' positions of the current chunk, in two rounds of two
    // loads: ranks by one packed DPP scan of the two loads' counts (16-bit
    // fields: at most 1024 each), positions staged at their ranks, then one
    // run to idx[seg + done ..).
    const auto write = [&](const uint32_t(&m)[kFlagMasks], int64_t chunk, uint32_t seg, int ln) {
        uint32_t done = 0;
#pragma unroll
        for (int q = 0; q < kFlagMasks; ++q) {
            const uint32_t mq = m[q];
            const uint32_t c = static_cast<uint32_t>(__builtin_popcount(mq & 0xFFFFu)) |
                               (static_cast<uint32_t>(__builtin_popcount(mq >> 16)) << 16);
            const uint32_t incl = wave_inclusive_scan<SumU32>(c);
            const uint32_t ex = incl - c;
            const uint32_t last = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
            const uint32_t t0 = last & 0xFFFFu;
            uint32_t r0 = ex & 0xFFFFu;
            uint32_t r1 = t0 + (ex >> 16);
            // positions of flags past n are formed but never staged: unsigned
            const uint32_t p0 = static_cast<uint32_t>(chunk) + static_cast<uint32_t>(2 * q * (kWave * 16) + ln * 16);
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const uint32_t f0 = (mq >> b) & 1u;
                const uint32_t f1 = (mq >> (16 + b)) & 1u;
                if (f0) s_stage[w][r0] = p0 + static_cast<uint32_t>(b);
                if (f1) s_stage[w][r1] = p0 + static_cast<uint32_t>(kWave * 16 + b);
                r0 += f0;
                r1 += f1;
            }
            const uint32_t len = t0 + (last >> 16);
            stream_run<kStageWords, kNT, true>(s_stage[w], reinterpret_cast<uint32_t *>(idx), seg + done,
                                               len, n, ln);
            done += len;
        }
    };

    u32x4 ra[kFlagLoads], rb[kFlagLoads];  // raw flags of the two tiles in flight
    uint32_t mc[kFlagMasks], mn[kFlagMasks];  // masks of the current and the next tile

    // One tile: X holds the next tile's flags, Y the tile after next's (in
    // flight); once X's masks are taken, X takes the loads of the tile the
    // control wavefront claimed during this one.
#define SSC_FLAG_TILE(X)                                                                      \
    {                                                                                         \
        int ln = lane;                                                                        \
        asm volatile("" : "+v"(ln));                                                          \
        const uint32_t tri_n = tri == 2u ? 0u : tri + 1u;                                     \
        arrive(masks(X, rem_of(nxt), ln, mn), nxt, tri_n, ln);                                \
        __syncthreads(); /* B1: this tile's base is known */                                  \
        const uint32_t nxt3 = uniform(s_next[par]);                                           \
        load(nxt3, ln, X);                                                                    \
        write(mc, chunk_of(tile), uniform(s_base[par]) + uniform(s_pre[tri][w]), ln);         \
        _Pragma("unroll") for (int q = 0; q < kFlagMasks; ++q) mc[q] = mn[q];                          \
        tile = nxt;                                                                           \
        nxt = nxt2;                                                                           \
        nxt2 = nxt3;                                                                          \
        par ^= 1u;                                                                            \
        tri = tri_n;                                                                          \
    }

    load(tile, lane, ra);
    __syncthreads();  // B0b: the second and third tiles
    uint32_t nxt = uniform(s_first[1]);
    uint32_t nxt2 = uniform(s_first[2]);
    load(nxt, lane, rb);
    arrive(masks(ra, rem_of(tile), lane, mc), tile, tri, lane);
    load(nxt2, lane, ra);
    __syncthreads();  // B0': every wavefront has arrived for the first tile
    while (true) {
        SSC_FLAG_TILE(rb)
        if (tile >= num_tiles) break;
        SSC_FLAG_TILE(ra)
        if (tile >= num_tiles) break;
    }
#undef SSC_FLAG_TILE
}

// =========================================================== scan kernel ---
constexpr int kScanPollSleep = 127;  // look-back poll interval, s_sleep units (measured)
// Exclusive (or, INCL, inclusive) scan of 32-bit values: one tile per
// workgroup, two workgroups resident per compute unit, with a control
// wavefront for the look-back (used for one to two tiles per compute unit;
// scan_persistent_kernel otherwise); the tile aggregate is
// the sum of the values. Per load j a lane sums its 4 values, a DPP wavefront
// scan gives the lane offsets, and results leave with the same 128-bit layout
// they were read with. in == out is allowed.
//
// WIDE (fp32 only): carries between tiles travel in fp64 (wide descriptors,
// fp64 look-back), and each output is rounded to fp32 once, from
// base + chunk prefix + the value's prefix inside its chunk, all added in
// fp64. Only the prefix inside a tile (at most 30720 values) is summed in
// fp32, so the error no longer grows with the number of tiles before.
template <class Op, bool VEC, bool INCL, bool WIDE>
__global__ __launch_bounds__(kLbBlock) __attribute__((amdgpu_waves_per_eu(8, 8))) void scan_kernel(const typename Op::T *in,
                                                        typename Op::T *out, int64_t n,
                                                        void *scratch, uint32_t num_tiles,
                                                        uint32_t capacity, typename Op::T *total) {
    using T = typename Op::T;
    __shared__ uint32_t s_tot[kChunksPerTile];
    __shared__ uint32_t s_pre[kChunksPerTile + 1];
    __shared__ uint32_t s_tile, s_tag, s_base, s_arrive;
    __shared__ double s_base64;
    static_assert(!WIDE || sizeof(typename Op::T) == 4, "wide carries are for fp32 values");

    const ScratchView sv = view(scratch);
    if (threadIdx.x == 0) {
        // the stale-slot sweep must spare every descriptor word this call uses
        const uint64_t c = claim_tile(sv, WIDE ? 2 * num_tiles : num_tiles, num_tiles, capacity);
        s_tile = static_cast<uint32_t>(c);
        s_tag = static_cast<uint32_t>(c >> 32) & kTagMask;
        s_arrive = 0;
    }
    __syncthreads();
    const uint32_t tile = uniform(s_tile);
    const uint32_t tag = uniform(s_tag);
    if (tile >= num_tiles) return;  // only if the scratch was never initialised
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t tile_start = static_cast<int64_t>(tile) * kTile;

    if (w == kCtrlWave) {
        if constexpr (WIDE) {
            double prefix = 0.0;
            if (tile != 0) prefix = look_back_wide<kScanPollSleep>(sv.desc, tile, tag, sv.timed_out);
            if (lane == 0) s_base64 = prefix;
            __syncthreads();  // B1
            T chunk_before[kLbRounds];
            T round_before[kLbRounds + 1];
            tile_prefixes<Op>(s_pre, 0, chunk_before, round_before);
            const double incl = prefix + static_cast<double>(round_before[kLbRounds]);
            if (lane == 0) {
                if (tile != 0) publish_wide(sv.desc, tile, tag, kStatusInclusive, incl);
                if (total != nullptr && tile == num_tiles - 1) *total = static_cast<T>(incl);
            }
        } else {
            T prefix = Op::zero();
            if (tile != 0) prefix = look_back<Op, kScanPollSleep>(sv.desc, tile, tag, sv.timed_out);
            if (lane == 0) s_base = Op::bits(prefix);
            __syncthreads();  // B1
            T chunk_before[kLbRounds];
            T round_before[kLbRounds + 1];
            tile_prefixes<Op>(s_pre, 0, chunk_before, round_before);
            const T agg = round_before[kLbRounds];
            if (lane == 0) {
                if (tile != 0)
                    publish(sv.desc + tile, tag, kStatusInclusive, Op::bits(Op::add(prefix, agg)));
                if (total != nullptr && tile == num_tiles - 1) *total = Op::add(prefix, agg);
            }
        }
        return;
    }

    T v[kLbRounds][kLoads][4];
#pragma unroll
    for (int q = 0; q < kLbRounds; ++q) {
        const int64_t chunk = tile_start + q * kLbSub + w * kChunk;
        load_chunk<VEC>(in, chunk, lane, chunk_rem(n, chunk), v[q]);  // missing read as 0
    }
    // Replace each value by its exclusive prefix inside the chunk.
#pragma unroll
    for (int q = 0; q < kLbRounds; ++q) {
        T running = Op::zero();
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            T s = Op::zero();
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const T x = v[q][j][k];
                if constexpr (INCL) {
                    s = Op::add(s, x);
                    v[q][j][k] = s;
                } else {
                    v[q][j][k] = s;
                    s = Op::add(s, x);
                }
            }
            const T incl = wave_inclusive_scan<Op>(s);
            const uint32_t up =
                static_cast<uint32_t>(__shfl_up(static_cast<int>(Op::bits(incl)), 1));
            const T lead = Op::add(running, lane == 0 ? Op::zero() : Op::from_bits(up));
#pragma unroll
            for (int k = 0; k < 4; ++k) v[q][j][k] = Op::add(lead, v[q][j][k]);
            running = Op::add(running, Op::from_bits(static_cast<uint32_t>(
                                           __builtin_amdgcn_readlane(
                                               static_cast<int>(Op::bits(incl)), kWave - 1))));
        }
        if (lane == 0) s_tot[q * kDataWaves + w] = Op::bits(running);
    }
    arrive_and_publish<Op, WIDE>(&s_arrive, s_tot, s_pre, sv.desc, tile, tag, lane);
    __syncthreads();  // B1
    T chunk_before[kLbRounds];
    T round_before[kLbRounds + 1];
    tile_prefixes<Op>(s_pre, w, chunk_before, round_before);
    const T base = Op::from_bits(uniform(s_base));
    const double base64 = WIDE ? s_base64 : 0.0;
#pragma unroll
    for (int q = 0; q < kLbRounds; ++q) {
        if constexpr (WIDE) {
            const double chunk_base = base64 + static_cast<double>(chunk_before[q]);
#pragma unroll
            for (int j = 0; j < kLoads; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[q][j][k] = static_cast<T>(chunk_base + static_cast<double>(v[q][j][k]));
        } else {
            const T chunk_base = Op::add(base, chunk_before[q]);
#pragma unroll
            for (int j = 0; j < kLoads; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k) v[q][j][k] = Op::add(chunk_base, v[q][j][k]);
        }
        const int64_t chunk = tile_start + q * kLbSub + w * kChunk;
        store_chunk<VEC>(out, chunk, lane, chunk_rem(n, chunk), v[q]);
    }
}

// ================================================== persistent scan kernel ---
// The scan in the compaction kernel's pipeline: one 1024-thread workgroup per
// compute unit loops over tiles of 30720 values claimed three ahead, each data
// wavefront holding three chunks of 2048 values (eight 128-bit loads per
// lane) in registers and parking one more in its 8 KiB LDS region. Per tile
// it
//   1. sums the next tile's chunk once it has landed and arrives with the
//      total; the last of the 15 to arrive scans the chunk totals and
//      publishes the next tile's {aggregate} at once;
//   2. issues the loads of the tile after next into the chunk parked last
//      (issued after the next tile's have landed, not before: fewer reads
//      waiting, 2^28 371.4 -> 367.4 us, fp32 377.4 -> 374.8);
//   3. waits at the tile's barrier, which hands over the base of the tile
//      before it (not of this one);
//   4. scans the previous tile's parked chunk load by load (per load a DPP
//      wavefront scan of the lanes' 4-value sums), stores base + chunk
//      prefix + the value's prefix in the layout it was read with, and parks
//      the current chunk in the same LDS bytes.
// So each look-back has a whole tile period: the control wavefront walks
// the look-back of the previous tile while the data wavefronts arrive for
// the next one, and publishes that tile's {inclusive} before the barrier.
// A workgroup passes one more barrier than it has tiles, for the base of its
// last one. Writing each chunk one barrier later took 2^28 from 367.0 to
// 358.9 us (fp32 372.2 -> 370.1); before it, the control wavefront was last
// at the barrier in 90% of the tiles and the data wavefronts waited there
// 3-5 us per tile. Scanning a chunk in place on arrival instead (its
// prefixes then live beside three register sets) spilled 8-39 dwords.
// WIDE (fp32): carries between tiles are fp64 (wide descriptors, fp64
// look-back) and each output is rounded to fp32 once from the fp64 sum of
// base, chunk prefix and in-chunk prefix. Forward progress as for
// select_kernel: a tile's aggregate waits only on its own data, and a
// look-back only on lower tiles. Earlier measurements (interleaved A/B,
// exclusive int32, before the parked chunk): 2^28 369.7 us against 377.1 for
// one workgroup per tile, fp32 376 against 405, 2^24 29.8 against 36.1.
constexpr int kScanPSleep = 32;  // look-back poll interval, s_sleep units

template <class Op, bool VEC, bool INCL, bool WIDE>
__global__ __launch_bounds__(kLbBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void scan_persistent_kernel(
    const typename Op::T *in, typename Op::T *out, int64_t n, void *scratch, uint32_t num_tiles,
    uint32_t capacity, typename Op::T *total) {
    using T = typename Op::T;
    using S = ChunkShape<kTileLoads, 4>;
    static_assert(S::kTileElems == kSelTile, "the compaction kernel's tile");
    static_assert(!WIDE || sizeof(T) == 4, "wide carries are for fp32 values");
    __shared__ uint32_t s_tot[kDataWaves];
    __shared__ uint32_t s_pre[3][kDataWaves + 1];  // chunk prefixes + aggregate, by tile mod 3
    __shared__ uint32_t s_base[2], s_next[2];      // by tile parity
    __shared__ double s_base64[2];
    __shared__ uint32_t s_first[3], s_epoch, s_arrive;
    __shared__ __attribute__((aligned(16))) uint32_t s_park[kDataWaves][S::kChunk];

    const ScratchView sv = view(scratch);
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    // descriptor words this call uses: the stale-slot sweep spares them
    const uint32_t words_used = WIDE ? 2u * num_tiles : num_tiles;
    if (threadIdx.x == 0) {
        const uint64_t c = claim_tiles(sv, 1);
        s_first[0] = static_cast<uint32_t>(c);
        s_epoch = static_cast<uint32_t>(c >> 32);
        s_arrive = 0;
    }
    __syncthreads();  // B0: the first tile
    uint32_t tile = uniform(s_first[0]);
    const uint32_t epoch = uniform(s_epoch);
    const uint32_t tag = epoch & kTagMask;
    if (tile >= num_tiles) {
        if (w == kCtrlWave && lane == 0) finish_claims(sv, epoch, gridDim.x, words_used, capacity);
        return;
    }
    bool last_claim = false;
    if (w == kCtrlWave && lane == 0) last_claim = claim_second_third(sv, num_tiles, s_first);
    uint32_t par = 0;
    uint32_t tri = 0;

    if (w == kCtrlWave) {
        __syncthreads();  // B0b: the second and third tiles
        uint32_t nxt = uniform(s_first[1]);
        uint32_t nxt2 = uniform(s_first[2]);
        __syncthreads();  // B0': the first tile's arrivals are in
        uint32_t prev = kNoTile;  // the tile whose base this iteration's barrier hands over
        while (true) {
            uint32_t nxt3 = kNoTile;
            if (lane == 0 && nxt2 < num_tiles) {
                nxt3 = static_cast<uint32_t>(claim_tiles(sv, 1));
                last_claim = nxt3 >= num_tiles;
            }
            if (prev != kNoTile) {
                T prefix = Op::zero();
                double prefix64 = 0.0;
                if (prev != 0) {
                    if constexpr (WIDE)
                        prefix64 = look_back_wide<kScanPSleep, false>(sv.desc, prev, tag, sv.timed_out);
                    else
                        prefix = look_back<Op, kScanPSleep, false>(sv.desc, prev, tag, sv.timed_out);
                }
                // prev's aggregate is read before the barrier: the arrivals of
                // the next iteration rewrite its slot
                const T agg = Op::from_bits(uniform(s_pre[tri == 0u ? 2u : tri - 1u][kDataWaves]));
                if (lane == 0) {
                    // {inclusive} two barriers after this tile's {aggregate}
                    if constexpr (WIDE) {
                        s_base64[par ^ 1u] = prefix64;
                        const double incl = prefix64 + static_cast<double>(agg);
                        if (prev != 0) publish_wide(sv.desc, prev, tag, kStatusInclusive, incl);
                        if (total != nullptr && prev == num_tiles - 1) *total = static_cast<T>(incl);
                    } else {
                        s_base[par ^ 1u] = Op::bits(prefix);
                        const T incl = Op::add(prefix, agg);
                        if (prev != 0) publish(sv.desc + prev, tag, kStatusInclusive, Op::bits(incl));
                        if (total != nullptr && prev == num_tiles - 1) *total = incl;
                    }
                }
            }
            if (lane == 0) s_next[par] = nxt3;
            __syncthreads();  // B1
            if (lane == 0) {
                if (last_claim) finish_claims(sv, epoch, gridDim.x, words_used, capacity);
                last_claim = false;
            }
            if (tile >= num_tiles) return;  // that barrier handed over this workgroup's last base
            prev = tile;
            tile = nxt;
            nxt = nxt2;
            nxt2 = uniform(nxt3);
            par ^= 1u;
            tri = tri == 2u ? 0u : tri + 1u;
        }
    }

    uint32_t va[S::kLoads][4], vb[S::kLoads][4], vc[S::kLoads][4];
    const auto chunk_of = [&](uint32_t t) {
        return static_cast<int64_t>(t) * S::kTileElems + static_cast<int64_t>(w) * S::kChunk;
    };
    const auto rem_of = [&](uint32_t t) {
        return t < num_tiles ? chunk_rem<S::kChunk>(n, chunk_of(t)) : 0u;
    };
    // Load j of a chunk goes through its own buffer resource, based j KiB
    // into the chunk with the bytes left from there: every lane then needs one
    // offset register, and the range check still covers the whole access
    // (the instruction's scalar offset is outside that check, so it cannot
    // carry j).
    // The byte count goes through readfirstlane: the compiler computes the
    // saturating subtraction in a VGPR, and a resource it cannot prove
    // wave-uniform wraps every load and store in a one-pass waterfall loop
    // (readfirstlane x4, two compares, exec juggling: 57 such loops in the
    // int32 kernel, 226 in the 32-bit-access form).
    const auto part_rsrc = [&](const void *chunk, uint32_t bytes, int j) {
        const uint32_t skip = static_cast<uint32_t>(j) * (kWave * 16);
        return buffer_rsrc(static_cast<const char *>(chunk) + skip, uniform(bytes > skip ? bytes - skip : 0u));
    };
    const auto load = [&](uint32_t t, int ln, uint32_t(&v)[S::kLoads][4]) {
        const T *c = in + chunk_of(t);
        const uint32_t bytes = rem_of(t) * 4u;
#pragma unroll
        for (int j = 0; j < S::kLoads; ++j) {
            const __amdgpu_buffer_rsrc_t r = part_rsrc(c, bytes, j);
            if constexpr (VEC) {
                const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, ln * 16, 0, kNT);
#pragma unroll
                for (int k = 0; k < 4; ++k) v[j][k] = q[k];
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[j][k] = __builtin_amdgcn_raw_buffer_load_b32(r, ln * 16 + 4 * k, 0, kNT);
            }
        }
    };
    // The chunk's total (values past the end read as 0).
    const auto chunk_sum = [&](const uint32_t(&v)[S::kLoads][4]) {
        T s = Op::zero();
#pragma unroll
        for (int j = 0; j < S::kLoads; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) s = Op::add(s, Op::from_bits(v[j][k]));
        const T incl = wave_inclusive_scan<Op>(s);
        return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(Op::bits(incl)), kWave - 1));
    };
    // Arrival with the chunk total: the last data wavefront to arrive scans
    // the 15 totals into s_pre[TRI] (fixed order, so fp32 sums agree for every
    // reader) and publishes tile T's {aggregate} ({inclusive} for tile 0).
    const auto arrive = [&](uint32_t tot, uint32_t t, uint32_t tri_, int ln) {
        if (ln == 0) s_tot[w] = tot;
        perturb(t * 16u + w, 11);
        uint32_t before = 0;
        if (ln == 0)
            before = __hip_atomic_fetch_add(&s_arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (uniform(before) == kDataWaves - 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            const T mine = ln < kDataWaves ? Op::from_bits(s_tot[ln]) : Op::zero();
            const T incl = wave_inclusive_scan<Op>(mine);
            const uint32_t up = static_cast<uint32_t>(__shfl_up(static_cast<int>(Op::bits(incl)), 1));
            if (ln < kDataWaves) s_pre[tri_][ln] = ln == 0 ? Op::bits(Op::zero()) : up;
            const T agg = Op::from_bits(static_cast<uint32_t>(
                __builtin_amdgcn_readlane(static_cast<int>(Op::bits(incl)), kDataWaves - 1)));
            if (ln == 0) {
                s_arrive = 0;
                s_pre[tri_][kDataWaves] = Op::bits(agg);
                if (t < num_tiles) {
                    const uint32_t st = t == 0 ? kStatusInclusive : kStatusAggregate;
                    if constexpr (WIDE)
                        publish_wide(sv.desc, t, tag, st, static_cast<double>(agg));
                    else
                        publish(sv.desc + t, tag, st, Op::bits(agg));
                }
            }
        }
    };
    // A tile's chunk is parked in the wavefront's LDS region from the barrier
    // of its own iteration to the next one, which hands over its base.
    // write_park scans the parked chunk of tile tp load by load (exclusive,
    // or with INCL inclusive) and stores base + chunk prefix + in-chunk
    // prefix in the load layout, and parks cur in its place: each load's 16
    // bytes per lane are read back, scanned and stored before the same bytes
    // take cur's values. The tags leave out either half.
    const auto write_park = [&](auto write_tag, auto park_tag, const uint32_t(&cur)[S::kLoads][4],
                                uint32_t tp, uint32_t par_p, uint32_t tri_p, int ln) {
        constexpr bool kWrite = decltype(write_tag)::value;
        constexpr bool kPark = decltype(park_tag)::value;
        u32x4 *slot = reinterpret_cast<u32x4 *>(&s_park[w][0]) + ln;
        const T *c = out + chunk_of(tp);
        const uint32_t bytes = kWrite ? rem_of(tp) * 4u : 0u;
        double b64 = 0.0;
        T base = Op::zero();
        if constexpr (kWrite) {
            const T cb = Op::from_bits(uniform(s_pre[tri_p][w]));
            if constexpr (WIDE)
                b64 = s_base64[par_p] + static_cast<double>(cb);
            else
                base = Op::add(Op::from_bits(uniform(s_base[par_p])), cb);
        }
        T running = Op::zero();
#pragma unroll
        for (int j = 0; j < S::kLoads; ++j) {
            if constexpr (kWrite) {
                const u32x4 xv = slot[j * kWave];
                T p[4];
                T s = Op::zero();
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const T x = Op::from_bits(xv[k]);
                    if constexpr (INCL) {
                        s = Op::add(s, x);
                        p[k] = s;
                    } else {
                        p[k] = s;
                        s = Op::add(s, x);
                    }
                }
                const T incl = wave_inclusive_scan<Op>(s);
                const uint32_t up = static_cast<uint32_t>(__shfl_up(static_cast<int>(Op::bits(incl)), 1));
                const T lead = Op::add(running, ln == 0 ? Op::zero() : Op::from_bits(up));
                running = Op::add(running, Op::from_bits(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                                               static_cast<int>(Op::bits(incl)), kWave - 1))));
                uint32_t q[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const T pre = Op::add(lead, p[k]);
                    if constexpr (WIDE)
                        q[k] = Op::bits(static_cast<T>(b64 + static_cast<double>(pre)));
                    else
                        q[k] = Op::bits(Op::add(base, pre));
                }
                const __amdgpu_buffer_rsrc_t r = part_rsrc(c, bytes, j);
                if constexpr (VEC) {
                    u32x4 o;
                    o[0] = q[0];
                    o[1] = q[1];
                    o[2] = q[2];
                    o[3] = q[3];
                    __builtin_amdgcn_raw_buffer_store_b128(o, r, ln * 16, 0, kNT);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        __builtin_amdgcn_raw_buffer_store_b32(q[k], r, ln * 16 + 4 * k, 0, kNT);
                }
            }
            if constexpr (kPark) {
                u32x4 o;
                o[0] = cur[j][0];
                o[1] = cur[j][1];
                o[2] = cur[j][2];
                o[3] = cur[j][3];
                slot[j * kWave] = o;
            }
        }
    };

    // One tile: CUR holds the current tile's chunk (arrived, parked after the
    // barrier), NX the next one in flight, FREE the chunk parked one tile
    // ago. The barrier hands over the previous tile's base, whose parked
    // chunk goes out before CUR takes its place.
#define SSC_SCAN_TILE(CUR, NX, FREE, WRITE)                                                  \
    {                                                                                        \
        int ln = lane;                                                                       \
        asm volatile("" : "+v"(ln));                                                         \
        const uint32_t tri_n = tri == 2u ? 0u : tri + 1u;                                    \
        arrive(chunk_sum(NX), nxt, tri_n, ln);                                               \
        /* the tile after next's loads leave once the next tile's have landed */             \
        load(nxt2, ln, FREE);                                                                \
        __syncthreads(); /* B1: the previous tile's base is known */                         \
        const uint32_t nxt3 = uniform(s_next[par]);                                          \
        write_park(std::integral_constant<bool, WRITE>{}, std::true_type{}, CUR, prev,       \
                   par ^ 1u, tri == 0u ? 2u : tri - 1u, ln);                                 \
        prev = tile;                                                                         \
        tile = nxt;                                                                          \
        nxt = nxt2;                                                                          \
        nxt2 = nxt3;                                                                         \
        par ^= 1u;                                                                           \
        tri = tri_n;                                                                         \
    }

    load(tile, lane, va);
    __syncthreads();  // B0b: the second and third tiles
    uint32_t nxt = uniform(s_first[1]);
    uint32_t nxt2 = uniform(s_first[2]);
    load(nxt, lane, vb);
    arrive(chunk_sum(va), tile, tri, lane);
    __syncthreads();  // B0': every wavefront has arrived for the first tile
    uint32_t prev = kNoTile;
    SSC_SCAN_TILE(va, vb, vc, false)  // the first tile: nothing parked yet
    if (tile < num_tiles) {
        while (true) {
            SSC_SCAN_TILE(vb, vc, va, true)
            if (tile >= num_tiles) break;
            SSC_SCAN_TILE(vc, va, vb, true)
            if (tile >= num_tiles) break;
            SSC_SCAN_TILE(va, vb, vc, true)
            if (tile >= num_tiles) break;
        }
    }
    __syncthreads();  // B1 once more: the base of this workgroup's last tile
    write_park(std::true_type{}, std::false_type{}, va, prev, par ^ 1u, tri == 0u ? 2u : tri - 1u, lane);
#undef SSC_SCAN_TILE
}

// ======================================================= counting kernels ---
// Grid-stride over sub-tiles. Each workgroup reduces its flag count in LDS,
// adds it to one of kSpread accumulators (spreading the atomics over several
// addresses), then counts itself done; the last workgroup to finish sums the
// accumulators, writes the result and clears the accumulators and the done
// counter for the next call. Thread 0 does all of a workgroup's global
// atomics, so its acquire-release on the done counter orders them.
template <int P, bool VEC>
__global__ __launch_bounds__(kBlock) void count_kernel(const int32_t *__restrict__ in, int64_t n,
                                                       PredArgs pr, uint32_t num_subs,
                                                       void *scratch, int32_t *__restrict__ result) {
    __shared__ uint32_t s_cnt[kWaves];
    const ScratchView sv = view(scratch);
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    uint32_t acc = 0;
    const auto chunk_of = [&](uint32_t s) {
        return static_cast<int64_t>(s) * kSub + static_cast<int64_t>(w) * kChunk;
    };
    const auto rem_of = [&](uint32_t s) { return s < num_subs ? chunk_rem(n, chunk_of(s)) : 0u; };
    const auto count = [&](const int32_t(&v)[kLoads][4], uint32_t rem) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc += static_cast<uint32_t>(__builtin_popcountll(
                    ballot(in_chunk(rem, j, lane, k) && pred_eval<P>(v[j][k], pr))));
    };
    // The next sub-tile's loads leave before the current one is counted. Buffer
    // loads drop the lanes past the end (they read 0; the validity test
    // discards them), so every iteration issues the same loads.
    int32_t va[kLoads][4], vb[kLoads][4];
    uint32_t sub = blockIdx.x;
    load_b32x4<kLoads, VEC>(in, chunk_of(sub), rem_of(sub), lane, va);
    while (sub < num_subs) {
        const uint32_t s1 = sub + gridDim.x;
        load_b32x4<kLoads, VEC>(in, chunk_of(s1), rem_of(s1), lane, vb);
        count(va, rem_of(sub));
        if (s1 >= num_subs) break;
        const uint32_t s2 = s1 + gridDim.x;
        load_b32x4<kLoads, VEC>(in, chunk_of(s2), rem_of(s2), lane, va);
        count(vb, rem_of(s1));
        sub = s2;
    }
    if (lane == 0) s_cnt[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t total = 0;
        for (int i = 0; i < kWaves; ++i) total += s_cnt[i];
        if (total != 0)
            __hip_atomic_fetch_add(sv.acc + (blockIdx.x % kSpread), total, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t done =
            __hip_atomic_fetch_add(sv.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            // all loads first: one coherent round trip, not one per accumulator
            uint32_t part[kSpread];
#pragma unroll
            for (int i = 0; i < kSpread; ++i)
                part[i] = __hip_atomic_load(sv.acc + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t k = 0;
#pragma unroll
            for (int i = 0; i < kSpread; ++i) {
                k += part[i];
                __hip_atomic_store(sv.acc + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            *result = static_cast<int32_t>(k);
            __hip_atomic_store(sv.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// For every bit b, the number of keys whose bit b is clear, left in
// kept32[0..31] of the scratch (same last-workgroup protocol as above; the
// 32 per-bit accumulators are 32 different addresses).
template <bool VEC>
__global__ __launch_bounds__(kBlock) void bit_clear_count_kernel(const uint32_t *__restrict__ in,
                                                                 int64_t n, uint32_t num_subs,
                                                                 void *scratch) {
    __shared__ uint32_t s_cnt[kWaves][32];
    const ScratchView sv = view(scratch);
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    // Per lane, keys with bit b set. Packed counting: word q of `nib` holds
    // 4-bit counters for bits q, q+4, ..., q+28, so one shift, mask and add
    // per word counts all 32 bits of a key; eight keys (at most 8 per
    // counter) are then unpacked into `set`. Invalid slots count as 0.
    uint32_t set[32];
#pragma unroll
    for (int b = 0; b < 32; ++b) set[b] = 0;
    uint32_t valid = 0;  // keys of this wavefront's chunks (uniform)
    for (uint32_t sub = blockIdx.x; sub < num_subs; sub += gridDim.x) {
        const int64_t chunk = static_cast<int64_t>(sub) * kSub + static_cast<int64_t>(w) * kChunk;
        const uint32_t rem = chunk_rem(n, chunk);
        valid += rem;
        uint32_t v[kLoads][4];
        load_chunk<VEC>(in, chunk, lane, rem, v);
#pragma unroll
        for (int half = 0; half < kLoads / 2; ++half) {
            uint32_t nib[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 2 * half; j < 2 * half + 2; ++j) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t x = in_chunk(rem, j, lane, k) ? v[j][k] : 0u;
#pragma unroll
                    for (int q = 0; q < 4; ++q) nib[q] += (x >> q) & 0x11111111u;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int i = 0; i < 8; ++i) set[q + 4 * i] += (nib[q] >> (4 * i)) & 0xFu;
            }
        }
    }
#pragma unroll
    for (int b = 0; b < 32; ++b) {
        const uint32_t all = wave_inclusive_scan<SumU32>(set[b]);
        const uint32_t t = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(all), kWave - 1));
        if (lane == 0) s_cnt[w][b] = valid - t;  // keys with bit b clear
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int b = 0; b < 32; ++b) {
            uint32_t t = 0;
            for (int i = 0; i < kWaves; ++i) t += s_cnt[i][b];
            if (t != 0)
                __hip_atomic_fetch_add(sv.acc32 + b, t, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t done =
            __hip_atomic_fetch_add(sv.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            // all loads first: one coherent round trip, not one per bit
            uint32_t t[32];
#pragma unroll
            for (int b = 0; b < 32; ++b)
                t[b] = __hip_atomic_load(sv.acc32 + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int b = 0; b < 32; ++b) {
                __hip_atomic_store(sv.kept32 + b, t[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sv.acc32 + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __hip_atomic_store(sv.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ======================================== radix sort with 4-bit digits ---
// Each pass is a stable 16-way split of the keys by digit (x >> shift) & 15,
// done as three steps over tiles of 8192 keys (one 512-thread workgroup, 16
// keys per lane):
//   digit_count_kernel: cnt[d * tiles + t] = keys of tile t with digit d;
//   one exclusive scan of that digit-major table (scan_impl) turns it
//     into off[d * tiles + t] = number of keys that precede, in the output,
//     the first digit-d key of tile t (all keys of smaller digits, plus the
//     digit-d keys of earlier tiles);
//   digit_scatter_kernel: stable ranks inside the tile, the tile staged in
//     LDS in digit order, then 16 contiguous runs written out.
// Composing four 1-bit splits of bits shift..shift+3 gives the same order, so
// after pass p the keys are stably sorted by their low 4(p+1) bits.
constexpr int kRadixDigits = 16;
constexpr int kRadixPassesMax = 8;

__host__ __device__ constexpr int64_t radix_tiles_for(int64_t n) { return (n + kSub - 1) / kSub; }

template <bool VEC>
__global__ __launch_bounds__(kBlock) void digit_count_kernel(const uint32_t *__restrict__ in,
                                                             int64_t n, int shift,
                                                             uint32_t *__restrict__ cnt,
                                                             uint32_t tiles) {
    __shared__ uint32_t s_c[kWaves][kRadixDigits];
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    if (lane < kRadixDigits) s_c[w][lane] = 0;
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * kSub + static_cast<int64_t>(w) * kChunk;
    const uint32_t rem = chunk_rem(n, chunk);
    uint32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, rem, v);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (in_chunk(rem, j, lane, k))
                __hip_atomic_fetch_add(&s_c[w][(v[j][k] >> shift) & 15u], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    if (threadIdx.x < kRadixDigits) {
        uint32_t t = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) t += s_c[i][threadIdx.x];
        cnt[threadIdx.x * tiles + blockIdx.x] = t;
    }
}

// Stable 16-way split of one tile. Ranks: each wavefront first transposes
// its 1024 keys through LDS so that slot (j, k) of lane l holds key
// j*256 + k*64 + l of its chunk; slots then run in key order. Per slot, four
// ballots of the digit bits give every lane the mask of lanes holding its
// digit; its rank is the running count of that digit in the wavefront (16
// LDS counters, bumped by the last lane of each digit) plus the matching
// lanes below it. Wavefront offsets per digit and the tile's digit starts
// follow from the 8 x 16 counts.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void digit_scatter_kernel(const uint32_t *__restrict__ in,
                                                               uint32_t *__restrict__ out,
                                                               int64_t n, int shift,
                                                               const uint32_t *__restrict__ off,
                                                               uint32_t tiles) {
    __shared__ __attribute__((aligned(16))) uint32_t s_keys[kSub];  // transposes, then the staged tile
    __shared__ uint32_t s_run[kWaves][kRadixDigits];
    __shared__ uint32_t s_before[kWaves][kRadixDigits];
    __shared__ uint32_t s_start[kRadixDigits];
    __shared__ uint32_t s_obase[kRadixDigits];
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t tile_start = static_cast<int64_t>(blockIdx.x) * kSub;
    const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
    const uint32_t rem = chunk_rem(n, chunk);
    if (lane < kRadixDigits) s_run[w][lane] = 0;

    uint32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, rem, v);
    uint32_t *mine = s_keys + w * kChunk;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        u32x4 q;
        q[0] = v[j][0];
        q[1] = v[j][1];
        q[2] = v[j][2];
        q[3] = v[j][3];
        *reinterpret_cast<u32x4 *>(mine + j * (kWave * 4) + lane * 4) = q;
    }
    uint32_t x[kLoads * 4];
    uint32_t rk[kLoads * 4];
#pragma unroll
    for (int t = 0; t < kLoads * 4; ++t) x[t] = mine[(t >> 2) * (kWave * 4) + (t & 3) * kWave + lane];

#pragma unroll
    for (int t = 0; t < kLoads * 4; ++t) {
        const uint32_t e = static_cast<uint32_t>((t >> 2) * (kWave * 4) + (t & 3) * kWave + lane);
        const bool valid = e < rem;
        const uint32_t d = (x[t] >> shift) & 15u;
        uint64_t m = ballot(valid);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint64_t bb = ballot(valid && ((d >> b) & 1u));
            m &= ((d >> b) & 1u) ? bb : ~bb;
        }
        const uint32_t below = mbcnt64(m);
        const uint32_t same = static_cast<uint32_t>(__builtin_popcountll(m));
        const uint32_t run = s_run[w][d];
        rk[t] = run + below;
        if (valid && below + 1u == same) s_run[w][d] = run + same;
    }
    __syncthreads();
    if (w == 0) {
        uint32_t acc = 0;
        if (lane < kRadixDigits) {
#pragma unroll
            for (int i = 0; i < kWaves; ++i) {
                s_before[i][lane] = acc;
                acc += s_run[i][lane];
            }
        }
        const uint32_t start = wave_inclusive_scan<SumU32>(acc) - acc;
        if (lane < kRadixDigits) {
            s_start[lane] = start;
            s_obase[lane] = off[lane * tiles + blockIdx.x] - start;
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kLoads * 4; ++t) {
        const uint32_t e = static_cast<uint32_t>((t >> 2) * (kWave * 4) + (t & 3) * kWave + lane);
        if (e < rem) {
            const uint32_t d = (x[t] >> shift) & 15u;
            s_keys[s_start[d] + s_before[w][d] + rk[t]] = x[t];
        }
    }
    __syncthreads();
    const int64_t left = n - tile_start;
    const uint32_t len = left >= kSub ? static_cast<uint32_t>(kSub) : static_cast<uint32_t>(left);
    for (uint32_t i = threadIdx.x; i < len; i += kBlock) {
        const uint32_t y = s_keys[i];
        const uint32_t o = s_obase[(y >> shift) & 15u] + i;
        // a correct count table never trips this; a broken one gives wrong
        // results instead of stray writes. Default cache policy: the next
        // pass reads this output (measured 435 us a sort against 439 us with
        // nontemporal stores, 2^24 keys)
        if (static_cast<int64_t>(o) < n) out[o] = y;
    }
}

// ================================================ unordered (atomic) kernel ---
// Comparison only: no scan, no order. One sub-tile per workgroup.
// VARIANT 0: the workgroup reserves one slot range for all its survivors with
// a single atomic add; VARIANT 1: one atomic add per survivor. *count must
// be zero beforehand.
template <int P, bool VEC, int VARIANT>
__global__ __launch_bounds__(kBlock) void compact_atomic_kernel(const int32_t *__restrict__ in,
                                                                int32_t *__restrict__ out,
                                                                int64_t n, PredArgs pr,
                                                                int32_t *__restrict__ count) {
    __shared__ uint32_t s_tot[kWaves];
    __shared__ uint32_t s_slot;
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t chunk =
        static_cast<int64_t>(blockIdx.x) * kSub + static_cast<int64_t>(w) * kChunk;
    const uint32_t rem = chunk_rem(n, chunk);
    int32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, rem, v);
    if constexpr (VARIANT == 0) {
        uint32_t lead[kLoads];
        uint64_t fmask = 0;
        const uint32_t t = chunk_ranks<P>(v, lane, rem, pr, lead, fmask, 0);
        if (lane == 0) s_tot[w] = t;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t total = 0;
            for (int i = 0; i < kWaves; ++i) total += s_tot[i];
            s_slot = total ? static_cast<uint32_t>(__hip_atomic_fetch_add(
                                 count, static_cast<int32_t>(total), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT))
                           : 0u;
        }
        __syncthreads();
        uint32_t slot = s_slot;
        for (int i = 0; i < w; ++i) slot += s_tot[i];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            uint32_t r = slot + lead[j];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (bit(fmask, j * 4 + k)) {
                    if (r < n) out[r] = v[j][k];
                    ++r;
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (in_chunk(rem, j, lane, k) && pred_eval<P>(v[j][k], pr)) {
                    const int32_t slot = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT);
                    if (slot < n) out[slot] = v[j][k];
                }
            }
        }
    }
}

// ============================================================ copy kernel ---
// The measured ceiling beside the compaction ("Day 33 compaction.cu",
// copyInts): one 256-thread workgroup per 4096 elements, four 128-bit
// nontemporal buffer loads then four stores per lane (32-bit ones for arrays
// that are not 16-byte aligned), the resource cut at n. Small workgroups of
// one shot each keep the most reads in flight on this part: at 2^28 int32
// this shape measured 336-339 us against 379 us for 512-thread workgroups
// with pointer accesses, and persistent grids 358 us.
constexpr int kCopyBlock = 256;
constexpr int kCopyLoads = 4;
constexpr int kCopyTile = kCopyBlock * kCopyLoads * 4;  // elements per workgroup

template <bool VEC>
__global__ __launch_bounds__(kCopyBlock) void copy_kernel(const int32_t *__restrict__ in,
                                                          int32_t *__restrict__ out, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyTile;
    const int64_t left = n - base;
    const uint32_t bytes =
        left >= kCopyTile ? static_cast<uint32_t>(kCopyTile) * 4u : static_cast<uint32_t>(left) * 4u;
    const __amdgpu_buffer_rsrc_t ri = buffer_rsrc(in + base, bytes);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(out + base, bytes);
    const int off = static_cast<int>(threadIdx.x) * 16;
    if constexpr (VEC) {
        u32x4 v[kCopyLoads];
#pragma unroll
        for (int j = 0; j < kCopyLoads; ++j)
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(ri, j * (kCopyBlock * 16) + off, 0, kNT);
#pragma unroll
        for (int j = 0; j < kCopyLoads; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(v[j], ro, j * (kCopyBlock * 16) + off, 0, kNT);
    } else {
        uint32_t v[kCopyLoads][4];
#pragma unroll
        for (int j = 0; j < kCopyLoads; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[j][k] = __builtin_amdgcn_raw_buffer_load_b32(ri, j * (kCopyBlock * 16) + off + 4 * k, 0,
                                                               kNT);
#pragma unroll
        for (int j = 0; j < kCopyLoads; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                __builtin_amdgcn_raw_buffer_store_b32(v[j][k], ro, j * (kCopyBlock * 16) + off + 4 * k, 0,
                                                      kNT);
    }
}

// ============================== multi-launch pipelines (comparison only) ---
// The pages' own structure, ported to this hardware to measure what the
// single pass saves: the flags are written out, scanned by a tree of tile
// scans (each writes its tiles' exclusive prefixes and one total per tile;
// the totals are scanned by the next level) whose carries are added back
// level by level, and a last kernel scatters the survivors to out[rank]
// ("Day 33 compaction.cu": mark, scan, scatter in seven launches at its
// size; "Day 32 scan_2.cu": tile scan, scan of the tile sums, add the
// offsets). Tiles are 8192 elements: one 512-thread workgroup, 16 per lane
// in the (load, lane, component) layout of the streaming kernels.

// flags[i] = P(in[i]).
template <int P, bool VEC>
__global__ __launch_bounds__(kBlock) void mark_kernel(const int32_t *__restrict__ in,
                                                      int32_t *__restrict__ flags, int64_t n,
                                                      PredArgs pr) {
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t chunk =
        static_cast<int64_t>(blockIdx.x) * kSub + static_cast<int64_t>(w) * kChunk;
    const uint32_t rem = chunk_rem(n, chunk);
    int32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, rem, v);
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] = pred_eval<P>(v[j][k], pr) ? 1 : 0;
    store_chunk<VEC>(flags, chunk, lane, rem, v);
}

// Exclusive scan inside each 8192-element tile of `in` (uint32 wrap) into
// `out` (in == out allowed); sums[tile] = the tile's total.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void tile_scan_kernel(const uint32_t *in, uint32_t *out,
                                                           int64_t n, uint32_t *__restrict__ sums,
                                                           uint32_t *__restrict__ total) {
    __shared__ uint32_t s_wave[kWaves];
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t chunk =
        static_cast<int64_t>(blockIdx.x) * kSub + static_cast<int64_t>(w) * kChunk;
    const uint32_t rem = chunk_rem(n, chunk);
    uint32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, rem, v);
    uint32_t running = 0;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        uint32_t s = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t x = v[j][k];
            v[j][k] = s;
            s += x;
        }
        const uint32_t incl = wave_inclusive_scan<SumU32>(s);
        const uint32_t lead = running + incl - s;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] += lead;
        running += static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
    }
    if (lane == 0) s_wave[w] = running;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < w; ++i) before += s_wave[i];
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] += before;
    store_chunk<VEC>(out, chunk, lane, rem, v);
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < kWaves; ++i) t += s_wave[i];
        sums[blockIdx.x] = t;
        if (total != nullptr && gridDim.x == 1) *total = t;  // the top level: the grand total
    }
}

// out[i] += carries[i / 8192] (uint32 wrap).
template <bool VEC>
__global__ __launch_bounds__(kBlock) void add_carry_kernel(uint32_t *__restrict__ out, int64_t n,
                                                           const uint32_t *__restrict__ carries) {
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t chunk =
        static_cast<int64_t>(blockIdx.x) * kSub + static_cast<int64_t>(w) * kChunk;
    const uint32_t rem = chunk_rem(n, chunk);
    const uint32_t c = carries[blockIdx.x];
    uint32_t v[kLoads][4];
    load_chunk<VEC>(out, chunk, lane, rem, v);
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] += c;
    store_chunk<VEC>(out, chunk, lane, rem, v);
}

// out[rank[i]] = in[i] where P(in[i]) (the predicate evaluated again rather
// than read back); the element n - 1 also writes the count.
template <int P>
__global__ __launch_bounds__(kBlock) void scatter_kernel(const int32_t *__restrict__ in,
                                                         const int32_t *__restrict__ rank,
                                                         int32_t *__restrict__ out, int64_t n,
                                                         PredArgs pr, int32_t *__restrict__ count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        const int32_t x = in[i];
        const bool f = pred_eval<P>(x, pr);
        const int32_t r = rank[i];
        if (f && r >= 0 && static_cast<int64_t>(r) < n) out[r] = x;
        if (i == n - 1) *count = r + (f ? 1 : 0);
    }
}

// *flag = the scratch's look-back time-out word (one thread; a coherent load,
// so a flag set by any compute unit is seen).
__global__ void timed_out_kernel(const uint32_t *__restrict__ word, int32_t *__restrict__ flag) {
    if (threadIdx.x == 0)
        *flag = static_cast<int32_t>(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Clears `words` 32-bit words (a kernel rather than a memset node).
__global__ __launch_bounds__(kBlock) void clear_kernel(uint32_t *__restrict__ p, int64_t words) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < words;
         i += static_cast<int64_t>(gridDim.x) * kBlock)
        p[i] = 0u;
}

}  // namespace ssc

// Scratch of ssc_compact_i32_noalloc: a look-back scratch (header and two
// descriptor words per tile) for every n the C ABI accepts, 1,119,232 bytes,
// held on each GPU the library runs on until the process ends. In host code
// this name stands for the symbol only: its device address comes from
// hipGetSymbolAddress (noalloc_scratch below), once per device.
constexpr size_t kNoAllocScratchBytes =
    (ssc::kHeaderBytes + static_cast<size_t>(ssc::desc_words(INT32_MAX)) * sizeof(uint64_t) + 255) &
    ~static_cast<size_t>(255);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// ======================================================================
// Host side: argument checks and dispatch.
// ======================================================================
namespace {

using namespace ssc;

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return SSC_ERR_HIP;
}

#define SSC_TRY(expr)                  \
    do {                               \
        const int rc_ = (expr);        \
        if (rc_ != SSC_OK) return rc_; \
    } while (0)

// Compute units of the current device: the persistent compaction kernel
// runs one workgroup on each.
int compute_units(uint32_t *out) {
    static int cus[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev >= 0 && dev < 64 && cus[dev] > 0) {
        *out = static_cast<uint32_t>(cus[dev]);
        return SSC_OK;
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    if (c <= 0) return SSC_ERR_DEVICE;
    if (dev >= 0 && dev < 64) cus[dev] = c;
    *out = static_cast<uint32_t>(c);
    return SSC_OK;
}

// Per-device check that the current device is gfx950 with 64-lane waves.
int check_device() {
    static int state[64];  // 0 unknown, 1 ok, 2 wrong device
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev >= 0 && dev < 64 && state[dev] == 1) return SSC_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.warpSize == 64;
    if (dev >= 0 && dev < 64) state[dev] = ok ? 1 : 2;
    return ok ? SSC_OK : SSC_ERR_DEVICE;
}

bool overlap(const void *a, size_t abytes, const void *b, size_t bbytes) {
    if (a == nullptr || b == nullptr || abytes == 0 || bbytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_pred(int pred, int32_t pa, int32_t pb) {
    (void)pb;
    switch (pred) {
    case SSC_PRED_NONZERO:
    case SSC_PRED_ODD:
    case SSC_PRED_EVEN:
        return SSC_OK;
    case SSC_PRED_BIT_SET:
    case SSC_PRED_BIT_CLEAR:
        return (pa >= 0 && pa <= 31) ? SSC_OK : SSC_ERR_ARG;
    case SSC_PRED_MOD_LT:
        return pa >= 1 ? SSC_OK : SSC_ERR_ARG;
    default:
        return SSC_ERR_ARG;
    }
}

// fp32 predicates take any thresholds (NaN included: every comparison with
// it is false).
int check_pred_f32(int pred) {
    return pred >= SSC_PRED_F32_NONZERO && pred <= SSC_PRED_F32_IN ? SSC_OK : SSC_ERR_ARG;
}

int32_t f32_bits(float f) {
    int32_t b;
    memcpy(&b, &f, 4);
    return b;
}

// Arguments of a predicate as the kernels take them (see PredArgs); for
// MOD_LT the fp64 constants of the residue test for the modulus a >= 1.
PredArgs make_pred_args(int pred, int32_t pa, int32_t pb) {
    PredArgs p{pa, pb, 0.0, 0.0, 0.0};
    if (pred == SSC_PRED_MOD_LT) {
        p.inv = 1.0 / static_cast<double>(pa);
        p.half = 0.5 * p.inv;
        p.thr = static_cast<double>(pb) / static_cast<double>(pa);
    }
    return p;
}

int check_n(int64_t n) {
    if (n < 0) return SSC_ERR_ARG;
    if (n > INT32_MAX) return SSC_ERR_SIZE;
    // only the stress build's small tiles can need more descriptor words
    if (desc_words(n) > static_cast<int64_t>(kMaxTiles)) return SSC_ERR_SIZE;
    return SSC_OK;
}

// Header plus two 64-bit descriptor words per tile (the fp32 scans' wide
// descriptors; the other kernels use the first half of the array).
size_t scratch_need(int64_t n) {
    return kHeaderBytes + static_cast<size_t>(n > 0 ? desc_words(n) : 0) * sizeof(uint64_t);
}

int check_scratch(const void *scratch, size_t bytes, size_t need) {
    if (scratch == nullptr || !aligned(scratch, 8) || bytes < need) return SSC_ERR_SCRATCH;
    return SSC_OK;
}

// Descriptor slots the scratch holds (the stale-slot sweep stays inside them).
uint32_t capacity_of(size_t scratch_bytes) {
    const size_t slots = (scratch_bytes - kHeaderBytes) / sizeof(uint64_t);
    return slots > kMaxTiles ? kMaxTiles : static_cast<uint32_t>(slots);
}

int launched() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSC_OK : hip_fail(e);
}

int clear_words(void *p, int64_t words, hipStream_t s) {
    if (words <= 0) return SSC_OK;
    int64_t blocks = (words + kBlock - 1) / kBlock;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(clear_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                       static_cast<uint32_t *>(p), words);
    return launched();
}

uint32_t subs_for(int64_t n) { return static_cast<uint32_t>((n + kSub - 1) / kSub); }

uint32_t reduce_grid(int64_t n) {
    const uint32_t subs = subs_for(n);
    return subs < static_cast<uint32_t>(kReduceGrid) ? subs : static_cast<uint32_t>(kReduceGrid);
}

// ---- template dispatch on the predicate and the load width ----
// Predicates 0..5 act on int32 elements, 6..9 on fp32 ones; F32 says which
// family the (already validated) predicate belongs to.
template <template <int, bool> class F, bool F32 = false, class... A>
int dispatch_pred(int pred, bool vec, A... a) {
    if constexpr (F32) {
        switch (pred) {
        case SSC_PRED_F32_NONZERO: return vec ? F<6, true>::run(a...) : F<6, false>::run(a...);
        case SSC_PRED_F32_GT: return vec ? F<7, true>::run(a...) : F<7, false>::run(a...);
        case SSC_PRED_F32_LT: return vec ? F<8, true>::run(a...) : F<8, false>::run(a...);
        default: return vec ? F<9, true>::run(a...) : F<9, false>::run(a...);
        }
    } else {
        switch (pred) {
        case 0: return vec ? F<0, true>::run(a...) : F<0, false>::run(a...);
        case 1: return vec ? F<1, true>::run(a...) : F<1, false>::run(a...);
        case 2: return vec ? F<2, true>::run(a...) : F<2, false>::run(a...);
        case 3: return vec ? F<3, true>::run(a...) : F<3, false>::run(a...);
        case 4: return vec ? F<4, true>::run(a...) : F<4, false>::run(a...);
        default: return vec ? F<5, true>::run(a...) : F<5, false>::run(a...);
        }
    }
}

// Workgroups for the radix driver's chained splits: the fewest that still
// take the tiles in as many rounds as one per compute unit would, when that
// is a few rounds. At 2^24 keys a split has 547 tiles, 2.1 rounds on 256
// compute units; 183 workgroups of 3 tiles each leave no near-empty last
// round (a 32-pass sort 1,105 -> 1,060 us). Other kinds and sizes keep one
// workgroup per compute unit: the same grid measured mixed elsewhere (2^25
// odd compaction 45.2 -> 42.8 us but the 2^25 int32 scan 49.3 -> 50.6, at
// two rounds the 8,387,997-element partition 32.0 -> 34.9, at 35 rounds
// selection by flag bytes 145.3 -> 147.6).
uint32_t split_grid(uint32_t tiles, uint32_t slots) {
    if (tiles <= slots) return tiles;
    const uint32_t rounds = (tiles + slots - 1) / slots;
    return rounds <= 8 ? (tiles + rounds - 1) / rounds : slots;
}

// One launch of the persistent kernel for element format F and kind KIND:
// one workgroup per compute unit, at most one per tile.
template <class F, int P, int KIND, int FORM = kFormDefault>
int launch_select(const SelArgs &a, int64_t n, PredArgs pr, void *scratch, uint32_t capacity,
                  int32_t *count, int32_t *ranks, const int32_t *kept, hipStream_t s) {
    constexpr int64_t kTileElems = F::Shape::kTileElems;
    const uint32_t tiles = static_cast<uint32_t>((n + kTileElems - 1) / kTileElems);
    uint32_t slots = 0;
    SSC_TRY(compute_units(&slots));
    const dim3 grid(KIND == kPartitionCached ? split_grid(tiles, slots) : (tiles < slots ? tiles : slots));
    hipLaunchKernelGGL((select_kernel<F, P, KIND, FORM>), grid, dim3(kLbBlock), 0, s, a, n, pr, scratch,
                       tiles, capacity, count, ranks, kept);
    return launched();
}

// Or-ed into a kind: a MOD_LT(m, s) compaction or selection takes the dense
// form of the kernel when it is expected to keep at least three quarters of
// uniform input (4s >= 3m); see FORM in select_kernel. Only the speed
// depends on it.
constexpr int kDenseKind = 0x100;
inline int with_density(int kind, int pred, int32_t pa, int32_t pb) {
    const bool dense = pred == SSC_PRED_MOD_LT && (kind == kCompact || kind == kSelectIndex) &&
                       4 * static_cast<int64_t>(pb) >= 3 * static_cast<int64_t>(pa);
    return dense ? (kind | kDenseKind) : kind;
}

// 32-bit elements, predicate P on the element.
template <int P, bool VEC>
struct LaunchSelect {
    static int run(int kind, const int32_t *in, int32_t *out, int64_t n, PredArgs pr,
                   void *scratch, uint32_t capacity, int32_t *count, int32_t *ranks,
                   const int32_t *kept, hipStream_t s) {
        using F = FmtB32<VEC>;
        const SelArgs a{in, nullptr, out, nullptr};
        const bool dense = (kind & kDenseKind) != 0;
        switch (kind & ~kDenseKind) {
        case kPartition:
            return launch_select<F, P, kPartition>(a, n, pr, scratch, capacity, count, ranks, kept, s);
        case kCompactRanks:
            return launch_select<F, P, kCompactRanks>(a, n, pr, scratch, capacity, count, ranks,
                                                      kept, s);
        case kSelectIndex:
            if constexpr (P == 5)
                if (dense)
                    return launch_select<F, P, kSelectIndex, kFormDense>(a, n, pr, scratch, capacity,
                                                                         count, ranks, kept, s);
            return launch_select<F, P, kSelectIndex>(a, n, pr, scratch, capacity, count, ranks,
                                                     kept, s);
        default:
            if constexpr (P == 5)
                if (dense)
                    return launch_select<F, P, kCompact, kFormDense>(a, n, pr, scratch, capacity,
                                                                     count, ranks, kept, s);
            return launch_select<F, P, kCompact>(a, n, pr, scratch, capacity, count, ranks, kept, s);
        }
    }
};

// Key-value pairs, predicate P on the key.
template <int P, bool VEC>
struct LaunchPairs {
    static int run(const SelArgs &a, int64_t n, PredArgs pr, void *scratch, uint32_t capacity,
                   int32_t *count, hipStream_t s) {
        return launch_select<FmtPairs<VEC>, P, kCompact>(a, n, pr, scratch, capacity, count,
                                                         nullptr, nullptr, s);
    }
};

// 64-bit elements, predicate P (0..4) on the element's bits.
template <int P, bool VEC>
struct LaunchSelect64 {
    static int run(int kind, const SelArgs &a, int64_t n, PredArgs pr, void *scratch,
                   uint32_t capacity, int32_t *count, hipStream_t s) {
        if (kind == kSelectIndex)
            return launch_select<FmtB64<VEC>, P, kSelectIndex>(a, n, pr, scratch, capacity, count,
                                                               nullptr, nullptr, s);
        return launch_select<FmtB64<VEC>, P, kCompact>(a, n, pr, scratch, capacity, count, nullptr,
                                                       nullptr, s);
    }
};

// The 64-bit predicates: nonzero, odd, even, bit set, bit clear.
template <template <int, bool> class F, class... A>
int dispatch_pred64(int pred, bool vec, A... a) {
    switch (pred) {
    case 0: return vec ? F<0, true>::run(a...) : F<0, false>::run(a...);
    case 1: return vec ? F<1, true>::run(a...) : F<1, false>::run(a...);
    case 2: return vec ? F<2, true>::run(a...) : F<2, false>::run(a...);
    case 3: return vec ? F<3, true>::run(a...) : F<3, false>::run(a...);
    default: return vec ? F<4, true>::run(a...) : F<4, false>::run(a...);
    }
}

template <int P, bool VEC>
struct LaunchCount {
    static int run(const int32_t *in, int64_t n, PredArgs pr, void *scratch,
                   int32_t *result, hipStream_t s) {
        hipLaunchKernelGGL((count_kernel<P, VEC>), dim3(reduce_grid(n)), dim3(kBlock), 0, s, in, n,
                           pr, subs_for(n), scratch, result);
        return launched();
    }
};

template <int P, bool VEC>
struct LaunchAtomic {
    static int run(int variant, const int32_t *in, int32_t *out, int64_t n, PredArgs pr,
                   int32_t *count, hipStream_t s) {
        const uint32_t subs = subs_for(n);
        if (variant == 0)
            hipLaunchKernelGGL((compact_atomic_kernel<P, VEC, 0>), dim3(subs), dim3(kBlock), 0, s,
                               in, out, n, pr, count);
        else
            hipLaunchKernelGGL((compact_atomic_kernel<P, VEC, 1>), dim3(subs), dim3(kBlock), 0, s,
                               in, out, n, pr, count);
        return launched();
    }
};

// ---- multi-launch pipelines (comparison) ----
// Words of tile sums for every level of the tile-scan tree over n values,
// each level rounded up to 4 words so that every level starts 16-byte aligned.
int64_t multipass_level_words(int64_t tiles) { return (tiles + 3) & ~int64_t{3}; }

int64_t multipass_sum_words(int64_t n) {
    int64_t words = 0;
    for (int64_t m = n; m > 1;) {
        const int64_t tiles = (m + kSub - 1) / kSub;
        words += multipass_level_words(tiles);
        m = tiles;
    }
    return words < 4 ? 4 : words;
}

// Exclusive scan of n uint32 values by levels: tile scans down the tree of
// tile sums, then the carries added back on the way up. The top level's
// total goes to *total when given. Launches: 2 * levels - 1.
int multipass_scan(const uint32_t *in, uint32_t *out, int64_t n, uint32_t *sums, uint32_t *total,
                   bool vec, hipStream_t s) {
    const uint32_t tiles = static_cast<uint32_t>((n + kSub - 1) / kSub);
    if (vec)
        hipLaunchKernelGGL((tile_scan_kernel<true>), dim3(tiles), dim3(kBlock), 0, s, in, out, n,
                           sums, total);
    else
        hipLaunchKernelGGL((tile_scan_kernel<false>), dim3(tiles), dim3(kBlock), 0, s, in, out, n,
                           sums, total);
    SSC_TRY(launched());
    if (tiles == 1) return SSC_OK;
    // the sums are scanned in place by the next level (aligned: scratch is)
    SSC_TRY(multipass_scan(sums, sums, tiles, sums + multipass_level_words(tiles), total, true, s));
    if (vec)
        hipLaunchKernelGGL((add_carry_kernel<true>), dim3(tiles), dim3(kBlock), 0, s, out, n, sums);
    else
        hipLaunchKernelGGL((add_carry_kernel<false>), dim3(tiles), dim3(kBlock), 0, s, out, n, sums);
    return launched();
}

template <int P, bool VEC>
struct LaunchMark {
    static int run(const int32_t *in, int32_t *flags, int64_t n, PredArgs pr, hipStream_t s) {
        hipLaunchKernelGGL((mark_kernel<P, VEC>), dim3(subs_for(n)), dim3(kBlock), 0, s, in, flags,
                           n, pr);
        return launched();
    }
};

template <int P, bool VEC>
struct LaunchScatter {
    static int run(const int32_t *in, const int32_t *rank, int32_t *out, int64_t n, PredArgs pr,
                   int32_t *count, hipStream_t s) {
        const int64_t blocks = (n + kBlock - 1) / kBlock;
        const dim3 grid(static_cast<unsigned>(blocks < 8192 ? blocks : 8192));
        hipLaunchKernelGGL((scatter_kernel<P>), grid, dim3(kBlock), 0, s, in, rank, out, n, pr,
                           count);
        return launched();
    }
};

template <class Op, bool INCL>
int scan_impl(const typename Op::T *in, typename Op::T *out, int64_t n, typename Op::T *total,
              void *scratch, size_t scratch_bytes, hipStream_t s) {
    using T = typename Op::T;
    SSC_TRY(check_n(n));
    if (n > 0 && (in == nullptr || out == nullptr)) return SSC_ERR_ARG;
    if (!aligned(in, 4) || !aligned(out, 4) || (total && !aligned(total, 4))) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * sizeof(T);
    if (in != out && overlap(in, bytes, out, bytes)) return SSC_ERR_ALIAS;
    if (total && (overlap(total, sizeof(T), in, bytes) || overlap(total, sizeof(T), out, bytes)))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, scratch_need(n)));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        (total && overlap(scratch, scratch_bytes, total, sizeof(T))))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return total ? clear_words(total, 1, s) : SSC_OK;
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    const uint32_t cap = capacity_of(scratch_bytes);
    constexpr bool kWide = sizeof(T) == 4 && !std::is_integral<T>::value;  // fp32: fp64 carries
    uint32_t slots = 0;
    SSC_TRY(compute_units(&slots));
    const bool vec = aligned(in, 16) && aligned(out, 16);
    if (tiles > slots && tiles <= 2 * slots) {
        // One to two tiles per compute unit: one workgroup per tile, two
        // resident per compute unit, beats a persistent workgroup taking
        // its two tiles in turn (10^7 int32: 19.6 against 22.5 us).
        if (vec)
            hipLaunchKernelGGL((scan_kernel<Op, true, INCL, kWide>), dim3(tiles), dim3(kLbBlock), 0, s, in, out,
                               n, scratch, tiles, cap, total);
        else
            hipLaunchKernelGGL((scan_kernel<Op, false, INCL, kWide>), dim3(tiles), dim3(kLbBlock), 0, s, in,
                               out, n, scratch, tiles, cap, total);
        return launched();
    }
    // persistent: one workgroup per compute unit, tiles of the compaction
    // kernel's size (the same as kTile but in the stress build)
    const uint32_t ptiles = static_cast<uint32_t>((n + kSelTile - 1) / kSelTile);
    const dim3 grid(ptiles < slots ? ptiles : slots);
    if (vec)
        hipLaunchKernelGGL((scan_persistent_kernel<Op, true, INCL, kWide>), grid, dim3(kLbBlock), 0, s, in,
                           out, n, scratch, ptiles, cap, total);
    else
        hipLaunchKernelGGL((scan_persistent_kernel<Op, false, INCL, kWide>), grid, dim3(kLbBlock), 0, s, in,
                           out, n, scratch, ptiles, cap, total);
    return launched();
}

// 4-bit radix sort scratch: a scan scratch for the 16 x tiles count table,
// then the table itself.
size_t radix4_scan_part(int64_t n) {
    const int64_t entries = kRadixDigits * radix_tiles_for(n);
    return (scratch_need(entries) + 255) & ~static_cast<size_t>(255);
}

size_t radix4_scratch_need(int64_t n) {
    if (n <= 0) return kHeaderBytes;
    return radix4_scan_part(n) + static_cast<size_t>(kRadixDigits * radix_tiles_for(n)) * 4;
}

// The checks of a compaction's arrays and predicate (everything but the
// scratch), made before anything is enqueued.
template <bool F32>
int compact_arrays_ok(const int32_t *in, const int32_t *out, int64_t n, int pred, int32_t pa,
                      int32_t pb, const int32_t *count, const int32_t *ranks) {
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || out == nullptr))) return SSC_ERR_ARG;
    SSC_TRY(F32 ? check_pred_f32(pred) : check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(count, 4) || (ranks && !aligned(ranks, 4)))
        return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, out, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, out, bytes) ||
        (ranks && (overlap(ranks, bytes, in, bytes) || overlap(ranks, bytes, out, bytes) ||
                   overlap(ranks, bytes, count, 4))))
        return SSC_ERR_ALIAS;
    return SSC_OK;
}

template <bool F32>
int compact_impl(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa, int32_t pb,
                 int32_t *count, int32_t *ranks, void *scratch, size_t scratch_bytes,
                 void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(compact_arrays_ok<F32>(in, out, n, pred, pa, pb, count, ranks));
    const size_t bytes = static_cast<size_t>(n) * 4;
    SSC_TRY(check_scratch(scratch, scratch_bytes, scratch_need(n)));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        overlap(scratch, scratch_bytes, count, 4) ||
        (ranks && overlap(scratch, scratch_bytes, ranks, bytes)))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const bool vec = aligned(in, 16) && (ranks == nullptr || aligned(ranks, 16));
    const int kind = with_density(ranks ? kCompactRanks : kCompact, pred, pa, pb);
    return dispatch_pred<LaunchSelect, F32>(pred, vec, kind, in, out, n,
                                       make_pred_args(pred, pa, pb), scratch,
                                       capacity_of(scratch_bytes), count, ranks,
                                       static_cast<const int32_t *>(nullptr), s);
}

template <bool F32>
int select_index_impl(const int32_t *in, int32_t *idx, int64_t n, int pred, int32_t pa, int32_t pb,
                      int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || idx == nullptr))) return SSC_ERR_ARG;
    SSC_TRY(F32 ? check_pred_f32(pred) : check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(idx, 4) || !aligned(count, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, idx, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, idx, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, scratch_need(n)));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, idx, bytes) ||
        overlap(scratch, scratch_bytes, count, 4))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const int kind = with_density(kSelectIndex, pred, pa, pb);
    return dispatch_pred<LaunchSelect, F32>(pred, aligned(in, 16), kind, in, idx, n,
                                       make_pred_args(pred, pa, pb), scratch,
                                       capacity_of(scratch_bytes), count,
                                       static_cast<int32_t *>(nullptr),
                                       static_cast<const int32_t *>(nullptr), s);
}

template <bool F32>
int partition_impl(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa, int32_t pb,
                   int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || out == nullptr))) return SSC_ERR_ARG;
    SSC_TRY(F32 ? check_pred_f32(pred) : check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(count, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, out, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, out, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, scratch_need(n)));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        overlap(scratch, scratch_bytes, count, 4))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const bool vec = aligned(in, 16);
    const PredArgs pr = make_pred_args(pred, pa, pb);
    SSC_TRY((dispatch_pred<LaunchCount, F32>(pred, vec, in, n, pr, scratch, count, s)));
    return dispatch_pred<LaunchSelect, F32>(pred, vec, kPartition, in, out, n, pr, scratch,
                                       capacity_of(scratch_bytes), static_cast<int32_t *>(nullptr),
                                       static_cast<int32_t *>(nullptr),
                                       static_cast<const int32_t *>(count), s);
}

// Arrays of one call with their byte extents: any two that overlap, or a
// pointer below the required alignment, make the call fail.
struct Span {
    const void *p;
    size_t bytes;
};

template <size_t N>
bool spans_overlap(const Span (&a)[N]) {
    for (size_t i = 0; i < N; ++i)
        for (size_t j = i + 1; j < N; ++j)
            if (overlap(a[i].p, a[i].bytes, a[j].p, a[j].bytes)) return true;
    return false;
}

// The scratch checks of every persistent-kernel call: large enough, and
// apart from each array of the call.
template <size_t N>
int check_scratch_apart(void *scratch, size_t scratch_bytes, int64_t n, const Span (&a)[N]) {
    SSC_TRY(check_scratch(scratch, scratch_bytes, scratch_need(n)));
    for (size_t i = 0; i < N; ++i)
        if (overlap(scratch, scratch_bytes, a[i].p, a[i].bytes)) return SSC_ERR_ALIAS;
    return SSC_OK;
}

// Compaction or selection by flag bytes (values == nullptr: positions).
int flags_impl(const void *in, const uint8_t *flags, void *out, int64_t n, int32_t *count,
               void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool values = in != nullptr;
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (flags == nullptr || out == nullptr))) return SSC_ERR_ARG;
    if (!aligned(flags, 4) || !aligned(out, 4) || !aligned(count, 4) || (values && !aligned(in, 4)))
        return SSC_ERR_ARG;
    const size_t words = static_cast<size_t>(n) * 4;
    const Span arrays[] = {{flags, static_cast<size_t>(n)}, {out, words}, {count, 4},
                           {in, values ? words : 0}};
    if (spans_overlap(arrays)) return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch_apart(scratch, scratch_bytes, n, arrays));
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const SelArgs a{in, flags, out, nullptr};
    const PredArgs pr{0, 0, 0.0, 0.0, 0.0};
    const uint32_t cap = capacity_of(scratch_bytes);
    if (!values && aligned(flags, 16)) {
        const uint32_t tiles = static_cast<uint32_t>((n + kFlagTile - 1) / kFlagTile);
        uint32_t slots = 0;
        SSC_TRY(compute_units(&slots));
        hipLaunchKernelGGL(select_flags_kernel, dim3(tiles < slots ? tiles : slots), dim3(kLbBlock), 0, s,
                           flags, static_cast<int32_t *>(out), n, scratch, tiles, cap, count);
        return launched();
    }
    if (!values)
        return launch_select<FmtFlags<true, false>, 0, kSelectIndex>(a, n, pr, scratch, cap, count,
                                                                     nullptr, nullptr, s);
    if (aligned(in, 16))
        return launch_select<FmtFlags<true, true>, 0, kCompact>(a, n, pr, scratch, cap, count,
                                                                nullptr, nullptr, s);
    return launch_select<FmtFlags<false, true>, 0, kCompact>(a, n, pr, scratch, cap, count,
                                                             nullptr, nullptr, s);
}

template <bool F32>
int kv_impl(const int32_t *keys, const void *vals, int32_t *keys_out, void *vals_out, int64_t n,
            int pred, int32_t pa, int32_t pb, int32_t *count, void *scratch, size_t scratch_bytes,
            void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr ||
        (n > 0 && (keys == nullptr || vals == nullptr || keys_out == nullptr || vals_out == nullptr)))
        return SSC_ERR_ARG;
    SSC_TRY(F32 ? check_pred_f32(pred) : check_pred(pred, pa, pb));
    if (!aligned(keys, 4) || !aligned(vals, 4) || !aligned(keys_out, 4) || !aligned(vals_out, 4) ||
        !aligned(count, 4))
        return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    const Span arrays[] = {{keys, bytes}, {vals, bytes}, {keys_out, bytes}, {vals_out, bytes},
                           {count, 4}};
    if (spans_overlap(arrays)) return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch_apart(scratch, scratch_bytes, n, arrays));
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const bool vec = aligned(keys, 16) && aligned(vals, 16);
    return dispatch_pred<LaunchPairs, F32>(pred, vec, SelArgs{keys, vals, keys_out, vals_out}, n,
                                           make_pred_args(pred, pa, pb), scratch,
                                           capacity_of(scratch_bytes), count, s);
}

int check_pred64(int pred, int32_t bit) {
    switch (pred) {
    case SSC_PRED_NONZERO:
    case SSC_PRED_ODD:
    case SSC_PRED_EVEN:
        return SSC_OK;
    case SSC_PRED_BIT_SET:
    case SSC_PRED_BIT_CLEAR:
        return (bit >= 0 && bit <= 63) ? SSC_OK : SSC_ERR_ARG;
    default:
        return SSC_ERR_ARG;
    }
}

// Compaction (kind kCompact, out = elements) or selection (kSelectIndex,
// out = int32 positions) of 64-bit elements.
int i64_impl(int kind, const int64_t *in, void *out, int64_t n, int pred, int32_t bit,
             int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || out == nullptr))) return SSC_ERR_ARG;
    SSC_TRY(check_pred64(pred, bit));
    const size_t out_elem = kind == kSelectIndex ? 4 : 8;
    if (!aligned(in, 8) || !aligned(out, out_elem) || !aligned(count, 4)) return SSC_ERR_ARG;
    const Span arrays[] = {{in, static_cast<size_t>(n) * 8},
                           {out, static_cast<size_t>(n) * out_elem}, {count, 4}};
    if (spans_overlap(arrays)) return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch_apart(scratch, scratch_bytes, n, arrays));
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    return dispatch_pred64<LaunchSelect64>(pred, aligned(in, 16), kind,
                                           SelArgs{in, nullptr, out, nullptr}, n,
                                           make_pred_args(pred, bit, 0), scratch,
                                           capacity_of(scratch_bytes), count, s);
}

// The device address of `scratch` on the current device, fetched once per
// device with that device current and kept; the first fetch also zero-fills
// the array on `s` (a clearing kernel ordered before the call that needs it:
// the look-back keeps the scratch ready from then on).
std::mutex g_noalloc_mutex;
void *g_noalloc_ptr[64];

int noalloc_scratch(void **ptr, hipStream_t s) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= 64) return SSC_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    if (g_noalloc_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (p == nullptr) return SSC_ERR_HIP;
        SSC_TRY(clear_words(p, static_cast<int64_t>(kNoAllocScratchBytes / 4), s));
        g_noalloc_ptr[dev] = p;
    }
    *ptr = g_noalloc_ptr[dev];
    return SSC_OK;
}

}  // namespace

// ======================================================================
// C ABI
// ======================================================================
extern "C" {

int64_t ssc_tile_elems(void) { return kSelTile; }

size_t ssc_scratch_bytes(int64_t n) { return scratch_need(n < 0 ? 0 : n); }

size_t ssc_radix_sort_scratch_bytes(int64_t n) { return scratch_need(n < 0 ? 0 : n); }

int ssc_scratch_init(void *scratch, size_t scratch_bytes, void *stream) {
    if (scratch == nullptr || !aligned(scratch, 8) || scratch_bytes < kHeaderBytes)
        return SSC_ERR_SCRATCH;
    SSC_TRY(check_device());
    return clear_words(scratch, static_cast<int64_t>(scratch_bytes / 4),
                       static_cast<hipStream_t>(stream));
}

int ssc_exclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                           void *scratch, size_t scratch_bytes, void *stream) {
    return scan_impl<SumU32, false>(reinterpret_cast<const uint32_t *>(in), reinterpret_cast<uint32_t *>(out),
                             n, reinterpret_cast<uint32_t *>(total), scratch, scratch_bytes,
                             static_cast<hipStream_t>(stream));
}

int ssc_exclusive_scan_f32(const float *in, float *out, int64_t n, float *total, void *scratch,
                           size_t scratch_bytes, void *stream) {
    return scan_impl<SumF32, false>(in, out, n, total, scratch, scratch_bytes,
                             static_cast<hipStream_t>(stream));
}

int ssc_inclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                           void *scratch, size_t scratch_bytes, void *stream) {
    return scan_impl<SumU32, true>(reinterpret_cast<const uint32_t *>(in),
                                   reinterpret_cast<uint32_t *>(out), n,
                                   reinterpret_cast<uint32_t *>(total), scratch, scratch_bytes,
                                   static_cast<hipStream_t>(stream));
}

int ssc_inclusive_scan_f32(const float *in, float *out, int64_t n, float *total, void *scratch,
                           size_t scratch_bytes, void *stream) {
    return scan_impl<SumF32, true>(in, out, n, total, scratch, scratch_bytes,
                                   static_cast<hipStream_t>(stream));
}

int ssc_compact_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa, int32_t pb,
                    int32_t *count, int32_t *ranks, void *scratch, size_t scratch_bytes,
                    void *stream) {
    return compact_impl<false>(in, out, n, pred, pa, pb, count, ranks, scratch, scratch_bytes,
                               stream);
}

int ssc_compact_i32_noalloc(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                            int32_t pb, int32_t *count, int32_t *ranks, void *stream) {
    SSC_TRY(compact_arrays_ok<false>(in, out, n, pred, pa, pb, count, ranks));
    if (scratch_need(n) > kNoAllocScratchBytes) return SSC_ERR_SIZE;
    SSC_TRY(check_device());
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 0) return clear_words(count, 1, s);
    void *p = nullptr;
    SSC_TRY(noalloc_scratch(&p, s));
    return compact_impl<false>(in, out, n, pred, pa, pb, count, ranks, p, kNoAllocScratchBytes,
                               stream);
}

int ssc_compact_f32(const float *in, float *out, int64_t n, int pred, float a, float b,
                    int32_t *count, int32_t *ranks, void *scratch, size_t scratch_bytes,
                    void *stream) {
    return compact_impl<true>(reinterpret_cast<const int32_t *>(in), reinterpret_cast<int32_t *>(out),
                              n, pred, f32_bits(a), f32_bits(b), count, ranks, scratch,
                              scratch_bytes, stream);
}

int ssc_select_index_i32(const int32_t *in, int32_t *idx, int64_t n, int pred, int32_t pa,
                         int32_t pb, int32_t *count, void *scratch, size_t scratch_bytes,
                         void *stream) {
    return select_index_impl<false>(in, idx, n, pred, pa, pb, count, scratch, scratch_bytes, stream);
}

int ssc_select_index_f32(const float *in, int32_t *idx, int64_t n, int pred, float a, float b,
                         int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    return select_index_impl<true>(reinterpret_cast<const int32_t *>(in), idx, n, pred, f32_bits(a),
                                   f32_bits(b), count, scratch, scratch_bytes, stream);
}

int ssc_partition_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa, int32_t pb,
                      int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    return partition_impl<false>(in, out, n, pred, pa, pb, count, scratch, scratch_bytes, stream);
}

int ssc_partition_f32(const float *in, float *out, int64_t n, int pred, float a, float b,
                      int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    return partition_impl<true>(reinterpret_cast<const int32_t *>(in),
                                reinterpret_cast<int32_t *>(out), n, pred, f32_bits(a), f32_bits(b),
                                count, scratch, scratch_bytes, stream);
}

int ssc_compact_flags_b32(const void *in, const uint8_t *flags, void *out, int64_t n,
                          int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    if (n > 0 && in == nullptr) return SSC_ERR_ARG;
    return flags_impl(in, flags, out, n, count, scratch, scratch_bytes, stream);
}

int ssc_select_flags(const uint8_t *flags, int32_t *idx, int64_t n, int32_t *count,
                     void *scratch, size_t scratch_bytes, void *stream) {
    return flags_impl(nullptr, flags, idx, n, count, scratch, scratch_bytes, stream);
}

int ssc_compact_kv_i32(const int32_t *keys, const void *vals, int32_t *keys_out, void *vals_out,
                       int64_t n, int pred, int32_t pa, int32_t pb, int32_t *count,
                       void *scratch, size_t scratch_bytes, void *stream) {
    return kv_impl<false>(keys, vals, keys_out, vals_out, n, pred, pa, pb, count, scratch,
                          scratch_bytes, stream);
}

int ssc_compact_kv_f32(const float *keys, const void *vals, float *keys_out, void *vals_out,
                       int64_t n, int pred, float a, float b, int32_t *count, void *scratch,
                       size_t scratch_bytes, void *stream) {
    return kv_impl<true>(reinterpret_cast<const int32_t *>(keys), vals,
                         reinterpret_cast<int32_t *>(keys_out), vals_out, n, pred, f32_bits(a),
                         f32_bits(b), count, scratch, scratch_bytes, stream);
}

int ssc_compact_i64(const int64_t *in, int64_t *out, int64_t n, int pred, int32_t bit,
                    int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    return i64_impl(kCompact, in, out, n, pred, bit, count, scratch, scratch_bytes, stream);
}

int ssc_select_index_i64(const int64_t *in, int32_t *idx, int64_t n, int pred, int32_t bit,
                         int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    return i64_impl(kSelectIndex, in, idx, n, pred, bit, count, scratch, scratch_bytes, stream);
}

int ssc_count_if_i32(const int32_t *in, int64_t n, int pred, int32_t pa, int32_t pb,
                     int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && in == nullptr)) return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(count, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(count, 4, in, bytes)) return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, kHeaderBytes));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, count, 4))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    return dispatch_pred<LaunchCount>(pred, aligned(in, 16), in, n, make_pred_args(pred, pa, pb),
                                      scratch, count, s);
}

int ssc_compact_atomic_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                           int32_t pb, int32_t *count, int variant, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || out == nullptr))) return SSC_ERR_ARG;
    if (variant != 0 && variant != 1) return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(count, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, out, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, out, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    SSC_TRY(clear_words(count, 1, s));
    if (n == 0) return SSC_OK;
    return dispatch_pred<LaunchAtomic>(pred, aligned(in, 16), variant, in, out, n,
                                       make_pred_args(pred, pa, pb), count,
                                       s);
}

int ssc_radix_sort_u32(const uint32_t *in, uint32_t *out, uint32_t *tmp, int64_t n, void *scratch,
                       size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (n > 0 && (in == nullptr || out == nullptr || tmp == nullptr)) return SSC_ERR_ARG;
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(tmp, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if ((in != out && overlap(in, bytes, out, bytes)) || overlap(tmp, bytes, in, bytes) ||
        overlap(tmp, bytes, out, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, ssc_radix_sort_scratch_bytes(n)));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        overlap(scratch, scratch_bytes, tmp, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return SSC_OK;
    const ScratchView sv = view(scratch);
    const bool vec = aligned(in, 16) && aligned(out, 16) && aligned(tmp, 16);
    if (vec)
        hipLaunchKernelGGL((bit_clear_count_kernel<true>), dim3(reduce_grid(n)), dim3(kBlock), 0,
                           s, in, n, subs_for(n), scratch);
    else
        hipLaunchKernelGGL((bit_clear_count_kernel<false>), dim3(reduce_grid(n)), dim3(kBlock), 0,
                           s, in, n, subs_for(n), scratch);
    SSC_TRY(launched());
    const uint32_t cap = capacity_of(scratch_bytes);
    const uint32_t *src = in;
    for (int b = 0; b < 32; ++b) {
        uint32_t *dst = (b % 2 == 0) ? tmp : out;  // pass 31 lands in out
        const int32_t *kept = reinterpret_cast<const int32_t *>(sv.kept32 + b);
        // the next split reads this output: keep it in the caches
        const SelArgs sa{src, nullptr, dst, nullptr};
        const PredArgs pr = make_pred_args(SSC_PRED_BIT_CLEAR, b, 0);
        if (vec)
            SSC_TRY((launch_select<FmtB32<true>, 4, kPartitionCached>(sa, n, pr, scratch, cap, nullptr,
                                                                      nullptr, kept, s)));
        else
            SSC_TRY((launch_select<FmtB32<false>, 4, kPartitionCached>(sa, n, pr, scratch, cap,
                                                                       nullptr, nullptr, kept, s)));
        src = dst;
    }
    return SSC_OK;
}

size_t ssc_radix_sort4_scratch_bytes(int64_t n) { return radix4_scratch_need(n); }

int ssc_radix_sort4_u32(const uint32_t *in, uint32_t *out, uint32_t *tmp, int64_t n, int passes,
                        void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (passes < 1 || passes > kRadixPassesMax) return SSC_ERR_ARG;
    if (n > 0 && (in == nullptr || out == nullptr || tmp == nullptr)) return SSC_ERR_ARG;
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(tmp, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    // pass 0 writes tmp when passes is even, so only then may out be in
    if ((n > 0 && in == out && passes % 2 == 1) || (in != out && overlap(in, bytes, out, bytes)) ||
        overlap(tmp, bytes, in, bytes) || overlap(tmp, bytes, out, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, radix4_scratch_need(n)));
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        overlap(scratch, scratch_bytes, tmp, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return SSC_OK;
    const uint32_t tiles = static_cast<uint32_t>(radix_tiles_for(n));
    const int64_t entries = static_cast<int64_t>(kRadixDigits) * tiles;
    const size_t scan_bytes = radix4_scan_part(n);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(static_cast<char *>(scratch) + scan_bytes);
    const bool vec = aligned(in, 16) && aligned(out, 16) && aligned(tmp, 16);
    const uint32_t *src = in;
    for (int p = 0; p < passes; ++p) {
        uint32_t *dst = (passes - 1 - p) % 2 == 0 ? out : tmp;  // the last pass lands in out
        if (vec)
            hipLaunchKernelGGL((digit_count_kernel<true>), dim3(tiles), dim3(kBlock), 0, s, src, n,
                               4 * p, cnt, tiles);
        else
            hipLaunchKernelGGL((digit_count_kernel<false>), dim3(tiles), dim3(kBlock), 0, s, src, n,
                               4 * p, cnt, tiles);
        SSC_TRY(launched());
        SSC_TRY((scan_impl<SumU32, false>(cnt, cnt, entries, nullptr, scratch, scan_bytes, s)));
        if (vec)
            hipLaunchKernelGGL((digit_scatter_kernel<true>), dim3(tiles), dim3(kBlock), 0, s, src,
                               dst, n, 4 * p, cnt, tiles);
        else
            hipLaunchKernelGGL((digit_scatter_kernel<false>), dim3(tiles), dim3(kBlock), 0, s, src,
                               dst, n, 4 * p, cnt, tiles);
        SSC_TRY(launched());
        src = dst;
    }
    return SSC_OK;
}

size_t ssc_multipass_scratch_bytes(int64_t n) {
    return static_cast<size_t>(multipass_sum_words(n < 0 ? 0 : n)) * 4 + 256;
}

int ssc_exclusive_scan_multipass_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                                     void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (n > 0 && (in == nullptr || out == nullptr)) return SSC_ERR_ARG;
    if (!aligned(in, 4) || !aligned(out, 4) || (total && !aligned(total, 4))) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (in != out && overlap(in, bytes, out, bytes)) return SSC_ERR_ALIAS;
    if (total && (overlap(total, 4, in, bytes) || overlap(total, 4, out, bytes)))
        return SSC_ERR_ALIAS;
    if (scratch == nullptr || !aligned(scratch, 16) ||
        scratch_bytes < ssc_multipass_scratch_bytes(n))
        return SSC_ERR_SCRATCH;
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        (total && overlap(scratch, scratch_bytes, total, 4)))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return total ? clear_words(total, 1, s) : SSC_OK;
    return multipass_scan(reinterpret_cast<const uint32_t *>(in), reinterpret_cast<uint32_t *>(out),
                          n, static_cast<uint32_t *>(scratch), reinterpret_cast<uint32_t *>(total),
                          aligned(in, 16) && aligned(out, 16), s);
}

int ssc_compact_multipass_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa,
                              int32_t pb, int32_t *count, int32_t *ranks, void *scratch,
                              size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || ranks == nullptr || (n > 0 && (in == nullptr || out == nullptr)))
        return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(count, 4) || !aligned(ranks, 4))
        return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, out, bytes) || overlap(ranks, bytes, in, bytes) ||
        overlap(ranks, bytes, out, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, out, bytes) || overlap(count, 4, ranks, bytes))
        return SSC_ERR_ALIAS;
    if (scratch == nullptr || !aligned(scratch, 16) ||
        scratch_bytes < ssc_multipass_scratch_bytes(n))
        return SSC_ERR_SCRATCH;
    if (overlap(scratch, scratch_bytes, in, bytes) || overlap(scratch, scratch_bytes, out, bytes) ||
        overlap(scratch, scratch_bytes, ranks, bytes) || overlap(scratch, scratch_bytes, count, 4))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const PredArgs pr = make_pred_args(pred, pa, pb);
    const bool vec = aligned(in, 16) && aligned(ranks, 16);
    SSC_TRY(dispatch_pred<LaunchMark>(pred, vec, in, ranks, n, pr, s));
    SSC_TRY(multipass_scan(reinterpret_cast<const uint32_t *>(ranks),
                           reinterpret_cast<uint32_t *>(ranks), n, static_cast<uint32_t *>(scratch),
                           nullptr, aligned(ranks, 16), s));
    return dispatch_pred<LaunchScatter>(pred, true, in, static_cast<const int32_t *>(ranks), out, n,
                                        pr, count, s);
}

int ssc_copy_i32(const int32_t *in, int32_t *out, int64_t n, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (n > 0 && (in == nullptr || out == nullptr)) return SSC_ERR_ARG;
    if (!aligned(in, 4) || !aligned(out, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, out, bytes)) return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return SSC_OK;
    const dim3 grid(static_cast<unsigned>((n + kCopyTile - 1) / kCopyTile));
    if (aligned(in, 16) && aligned(out, 16))
        hipLaunchKernelGGL((copy_kernel<true>), grid, dim3(kCopyBlock), 0, s, in, out, n);
    else
        hipLaunchKernelGGL((copy_kernel<false>), grid, dim3(kCopyBlock), 0, s, in, out, n);
    return launched();
}

int ssc_scratch_timed_out(const void *scratch, size_t scratch_bytes, int32_t *flag, void *stream) {
    if (scratch == nullptr || !aligned(scratch, 8) || scratch_bytes < kHeaderBytes)
        return SSC_ERR_SCRATCH;
    if (flag == nullptr || !aligned(flag, 4)) return SSC_ERR_ARG;
    if (overlap(scratch, scratch_bytes, flag, 4)) return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    const ScratchView sv = view(const_cast<void *>(scratch));
    hipLaunchKernelGGL(timed_out_kernel, dim3(1), dim3(kWave), 0, static_cast<hipStream_t>(stream),
                       sv.timed_out, flag);
    return launched();
}

int ssc_mark_i32(const int32_t *in, int32_t *flags, int64_t n, int pred, int32_t pa, int32_t pb,
                 void *stream) {
    SSC_TRY(check_n(n));
    if (n > 0 && (in == nullptr || flags == nullptr)) return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(flags, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    if (overlap(in, bytes, flags, bytes)) return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return SSC_OK;
    return dispatch_pred<LaunchMark>(pred, aligned(in, 16) && aligned(flags, 16), in, flags, n,
                                     make_pred_args(pred, pa, pb), static_cast<hipStream_t>(stream));
}

int ssc_scatter_i32(const int32_t *in, const int32_t *ranks, int32_t *out, int64_t n, int pred,
                    int32_t pa, int32_t pb, int32_t *count, void *stream) {
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || ranks == nullptr || out == nullptr)))
        return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(ranks, 4) || !aligned(out, 4) || !aligned(count, 4))
        return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    const Span arrays[] = {{in, bytes}, {ranks, bytes}, {out, bytes}, {count, 4}};
    if (spans_overlap(arrays)) return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 0) return clear_words(count, 1, s);
    return dispatch_pred<LaunchScatter>(pred, true, in, ranks, out, n, make_pred_args(pred, pa, pb),
                                        count, s);
}

const char *ssc_status_str(int status) {
    switch (status) {
    case SSC_OK: return "ok";
    case SSC_ERR_ARG: return "invalid argument";
#ifdef SSC_STRESS_TILES
    case SSC_ERR_SIZE: return "n exceeds 2^17 tiles of 3840 elements (the small-tile test build's limit)";
#else
    case SSC_ERR_SIZE: return "n exceeds INT32_MAX";
#endif
    case SSC_ERR_ALIAS: return "buffers overlap";
    case SSC_ERR_SCRATCH: return "scratch too small or misaligned";
    case SSC_ERR_HIP: return "HIP error";
    case SSC_ERR_DEVICE: return "device is not gfx950 with 64-wide wavefronts";
    default: return "unknown status";
    }
}

int ssc_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
