// Single-pass scan, stream compaction and stable partition for MI355X
// (gfx950, CDNA4): HIP kernels and the C ABI declared in include/ssc.h.
//
// Method ("Day 33 compaction.cu", header comment; "CUDA Handbook ch. 13,
// Stream Compaction", Listings 13-17/13-18): flag each element with a
// predicate, exclusive-scan the flags, scatter survivors to out[rank]; the
// count is the top of the scan, and a partition sends rejected x[i] to
// out[K + i - rank[i]]. Here the whole path is one kernel launch over tiles
// whose numbers come from an atomic counter, each tile finding the number of
// survivors before it by a decoupled look-back over per-tile descriptors.
//
// Tile shape (MI355X-first, not the pages' 256- or 1024-thread blocks):
// a 256-thread workgroup = 4 wavefronts of 64 lanes; each wavefront owns a
// contiguous chunk of 64 * E elements and reads it with 128-bit loads, E/4
// per lane, every load instruction covering 1 KiB of consecutive bytes.
// Element order inside the chunk is (load j, lane, component k). Ranks inside
// a wavefront come from ballot + mbcnt (no shared-memory tree), wave totals
// meet in LDS, survivors are staged in LDS at their tile rank and leave as
// one contiguous run of coalesced stores.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "ssc.h"
#include "ssc_device.h"

namespace ssc {

// ------------------------------------------------------------ tile shape ---
constexpr int kBlock = 256;               // threads per workgroup
constexpr int kWaves = kBlock / kWave;    // 4 wavefronts
constexpr int kLoads = 4;                 // 128-bit loads per lane
constexpr int kItems = 4 * kLoads;        // 16 elements per lane
constexpr int kChunk = kWave * kItems;    // 1024 elements per wavefront
constexpr int kTile = kBlock * kItems;    // 4096 elements per tile
constexpr int kReduceGrid = 2048;         // workgroups of the grid-stride counting kernels

constexpr size_t kHeaderBytes = 256;       // tile counter, time-out flag
constexpr size_t kRadixHeaderBytes = 512;  // 32 tile counters, 32 bit counts, time-out flag

__host__ __device__ constexpr int64_t tiles_for(int64_t n) { return (n + kTile - 1) / kTile; }

// Four 32-bit lanes moved by one 128-bit global load or store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// --------------------------------------------------------------- loading ---
// Loads this lane's kItems elements of the chunk starting at `chunk`:
// v[j][k] = in[chunk + j*256 + lane*4 + k]. `full` (uniform) says the whole
// tile is in range; otherwise each element is checked against n and missing
// ones read as 0 with valid = false. VEC selects 128-bit loads (the array is
// 16-byte aligned) or 32-bit loads.
template <bool VEC, class T>
__device__ __forceinline__ void load_chunk(const T *__restrict__ in, int64_t chunk, int lane,
                                           int64_t n, bool full, T (&v)[kLoads][4]) {
    static_assert(sizeof(T) == 4, "32-bit elements");
    if (full) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
            if constexpr (VEC) {
                const u32x4 q = *reinterpret_cast<const u32x4 *>(in + at);
                v[j][0] = from_u32<T>(q[0]);
                v[j][1] = from_u32<T>(q[1]);
                v[j][2] = from_u32<T>(q[2]);
                v[j][3] = from_u32<T>(q[3]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) v[j][k] = in[at + k];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[j][k] = (at + k < n) ? in[at + k] : T(0);
        }
    }
}

template <bool VEC, class T>
__device__ __forceinline__ void store_chunk(T *out, int64_t chunk, int lane, int64_t n, bool full,
                                            const T (&v)[kLoads][4]) {
    if (full) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
            if constexpr (VEC) {
                u32x4 q;
                q[0] = to_u32(v[j][0]);
                q[1] = to_u32(v[j][1]);
                q[2] = to_u32(v[j][2]);
                q[3] = to_u32(v[j][3]);
                *reinterpret_cast<u32x4 *>(out + at) = q;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) out[at + k] = v[j][k];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (at + k < n) out[at + k] = v[j][k];
        }
    }
}

// Flags and wavefront-local ranks for one chunk. On return:
//   f[j][k]   = element valid and predicate true,
//   kb[j][k]  = number of flagged elements before (j, lane, k) in the chunk,
// and the chunk's flag total is returned (uniform).
template <int P>
__device__ __forceinline__ uint32_t chunk_ranks(const int32_t (&v)[kLoads][4], int64_t chunk,
                                                int lane, int64_t n, bool full, int32_t pa,
                                                int32_t pb, bool (&f)[kLoads][4],
                                                uint32_t (&kb)[kLoads][4]) {
    uint32_t running = 0;  // flagged elements in earlier loads of this chunk (uniform)
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int64_t at = chunk + j * (kWave * 4) + lane * 4;
        uint64_t m[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[j][k] = (full || at + k < n) && pred_eval<P>(v[j][k], pa, pb);
            m[k] = ballot(f[j][k]);
        }
        uint32_t below = 0;  // flagged elements of load j in lower lanes
        uint32_t total = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            below += mbcnt64(m[k]);
            total += static_cast<uint32_t>(__builtin_popcountll(m[k]));
        }
        uint32_t in_lane = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            kb[j][k] = running + below + in_lane;
            in_lane += f[j][k] ? 1u : 0u;
        }
        running += total;
    }
    return running;
}

// Sum of the wave totals below `w` and of all waves, after the barrier that
// published them in LDS.
__device__ __forceinline__ void wave_offsets(const uint32_t *s_tot, int w, uint32_t &below,
                                             uint32_t &all) {
    below = 0;
    all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t t = s_tot[i];
        below += (i < w) ? t : 0u;
        all += t;
    }
}

// ===================================================== compaction kernel ---
// One launch, one tile per workgroup (tile number from the atomic counter).
//   1. claim a tile, load it (128-bit loads), flag it, rank it per wavefront;
//   2. wave totals in LDS -> tile aggregate A and each wavefront's offset;
//   3. publish {aggregate, A} (tile 0 publishes {inclusive, A});
//   4. stage survivors in LDS at their tile rank (partition: rejected ones
//      after them at A + local index - rank) while wavefront 0 looks back;
//   5. publish {inclusive, base + A}; barrier; stream the staged run(s) out.
// PARTITION reads K from *kept_total (written by the counting pass).
template <int P, bool VEC, bool PARTITION>
__global__ __launch_bounds__(kBlock) void select_kernel(
    const int32_t *__restrict__ in, int32_t *__restrict__ out, int64_t n, int32_t pa,
    int32_t pb, uint64_t *__restrict__ desc, uint32_t *__restrict__ tile_counter,
    uint32_t *__restrict__ timed_out, uint32_t num_tiles, int32_t *__restrict__ count,
    int32_t *__restrict__ ranks, const int32_t *__restrict__ kept_total) {
    __shared__ int32_t s_stage[kTile];
    __shared__ uint32_t s_tot[kWaves];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_base;

    if (threadIdx.x == 0) s_tile = claim_tile(tile_counter);
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile >= num_tiles) return;  // only if the counter was not cleared
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t tile_start = static_cast<int64_t>(tile) * kTile;
    const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
    const bool full = tile_start + kTile <= n;

    int32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, n, full, v);

    bool f[kLoads][4];
    uint32_t kb[kLoads][4];
    const uint32_t wave_total = chunk_ranks<P>(v, chunk, lane, n, full, pa, pb, f, kb);
    if (lane == 0) s_tot[w] = wave_total;
    __syncthreads();
    uint32_t wave_below, agg;
    wave_offsets(s_tot, w, wave_below, agg);

    if (threadIdx.x == 0)
        publish(desc + tile, tile == 0 ? kStatusInclusive : kStatusAggregate, agg);

    // Stage: survivors at their tile rank; for a partition the rejected
    // elements follow at A + (local index - rank).
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t local = static_cast<uint32_t>(w * kChunk + j * (kWave * 4) + lane * 4 + k);
            const uint32_t r = wave_below + kb[j][k];
            if (f[j][k]) {
                s_stage[r] = v[j][k];
            } else if constexpr (PARTITION) {
                if (full || tile_start + local < n) s_stage[agg + local - r] = v[j][k];
            }
        }
    }

    if (w == 0) {
        uint32_t base = 0;
        if (tile != 0) {
            base = look_back<SumU32>(desc, tile, timed_out);
            if (lane == 0) publish(desc + tile, kStatusInclusive, base + agg);
        }
        if (lane == 0) {
            s_base = base;
            if (!PARTITION && tile == num_tiles - 1) *count = static_cast<int32_t>(base + agg);
        }
    }
    __syncthreads();
    const uint32_t base = s_base;

    if constexpr (!PARTITION) {
        // Range-checked: a correct look-back never trips it; a broken one
        // gives wrong results instead of stray writes.
        for (uint32_t i = threadIdx.x; i < agg; i += kBlock)
            if (base + i < n) out[base + i] = s_stage[i];
        if (ranks != nullptr) {
            int32_t rk[kLoads][4];
#pragma unroll
            for (int j = 0; j < kLoads; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    rk[j][k] = static_cast<int32_t>(base + wave_below + kb[j][k]);
            store_chunk<VEC>(ranks, chunk, lane, n, full, rk);
        }
    } else {
        const uint32_t kept = static_cast<uint32_t>(*kept_total);
        const uint32_t len = full ? kTile : static_cast<uint32_t>(n - tile_start);
        // rejected elements before this tile = tile_start - base
        const uint32_t rej_base = kept + static_cast<uint32_t>(tile_start) - base - agg;
        for (uint32_t i = threadIdx.x; i < len; i += kBlock) {
            const uint32_t dst = (i < agg ? base : rej_base) + i;
            if (dst < n) out[dst] = s_stage[i];
        }
    }
}

// =========================================================== scan kernel ---
// Exclusive scan of 32-bit values, same tile shape and look-back; the tile
// aggregate is the sum of the values. Per load j a lane sums its 4 values,
// a DPP wavefront scan gives the lane offsets, and the outputs are written
// back with the same 128-bit layout they were read with. in == out allowed.
template <class Op, bool VEC>
__global__ __launch_bounds__(kBlock) void scan_kernel(
    const typename Op::T *in, typename Op::T *out, int64_t n, uint64_t *__restrict__ desc,
    uint32_t *__restrict__ tile_counter, uint32_t *__restrict__ timed_out, uint32_t num_tiles,
    typename Op::T *total) {
    using T = typename Op::T;
    __shared__ uint32_t s_tot[kWaves];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_base;

    if (threadIdx.x == 0) s_tile = claim_tile(tile_counter);
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile >= num_tiles) return;  // only if the counter was not cleared
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t tile_start = static_cast<int64_t>(tile) * kTile;
    const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
    const bool full = tile_start + kTile <= n;

    T v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, n, full, v);  // missing elements read as 0

    // Per load: in-lane exclusive prefixes, lane offset within the wavefront,
    // and the wavefront-uniform running total of earlier loads.
    T lane_off[kLoads];
    T load_run[kLoads];
    T running = Op::zero();
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        T s = Op::zero();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const T x = v[j][k];
            v[j][k] = s;  // in-lane exclusive prefix
            s = Op::add(s, x);
        }
        const T incl = wave_inclusive_scan<Op>(s);
        const uint32_t up = static_cast<uint32_t>(
            __shfl_up(static_cast<int>(Op::bits(incl)), 1));
        lane_off[j] = lane == 0 ? Op::zero() : Op::from_bits(up);
        load_run[j] = running;
        const T load_total = Op::from_bits(static_cast<uint32_t>(
            __builtin_amdgcn_readlane(static_cast<int>(Op::bits(incl)), kWave - 1)));
        running = Op::add(running, load_total);
    }
    if (lane == 0) s_tot[w] = Op::bits(running);
    __syncthreads();
    T wave_below = Op::zero();
    T agg = Op::zero();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const T t = Op::from_bits(s_tot[i]);
        if (i < w) wave_below = Op::add(wave_below, t);
        agg = Op::add(agg, t);
    }
    if (threadIdx.x == 0)
        publish(desc + tile, tile == 0 ? kStatusInclusive : kStatusAggregate, Op::bits(agg));

    if (w == 0) {
        T base = Op::zero();
        if (tile != 0) {
            base = look_back<Op>(desc, tile, timed_out);
            if (lane == 0) publish(desc + tile, kStatusInclusive, Op::bits(Op::add(base, agg)));
        }
        if (lane == 0) {
            s_base = Op::bits(base);
            if (total != nullptr && tile == num_tiles - 1) *total = Op::add(base, agg);
        }
    }
    __syncthreads();
    const T chunk_base = Op::add(Op::from_bits(s_base), wave_below);

#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const T lead = Op::add(load_run[j], lane_off[j]);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] = Op::add(chunk_base, Op::add(lead, v[j][k]));
    }
    store_chunk<VEC>(out, chunk, lane, n, full, v);
}

// ======================================================= counting kernels ---
// Grid-stride over tiles; each wavefront adds popcount(ballot(flag)) and
// makes one atomic add at the end. *count must be zero beforehand.
template <int P, bool VEC>
__global__ __launch_bounds__(kBlock) void count_kernel(const int32_t *__restrict__ in, int64_t n,
                                                       int32_t pa, int32_t pb, uint32_t num_tiles,
                                                       int32_t *__restrict__ count) {
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    uint32_t acc = 0;
    for (uint32_t tile = blockIdx.x; tile < num_tiles; tile += gridDim.x) {
        const int64_t tile_start = static_cast<int64_t>(tile) * kTile;
        const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
        const bool full = tile_start + kTile <= n;
        int32_t v[kLoads][4];
        load_chunk<VEC>(in, chunk, lane, n, full, v);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool f = (full || at + k < n) && pred_eval<P>(v[j][k], pa, pb);
                acc += static_cast<uint32_t>(__builtin_popcountll(ballot(f)));
            }
        }
    }
    if (lane == 0 && acc != 0)
        __hip_atomic_fetch_add(count, static_cast<int32_t>(acc), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// For every bit b, the number of keys whose bit b is clear, added into
// clear_counts[0..31] (zero beforehand). Lane b carries bit b's total to one
// atomic add per wavefront.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void bit_clear_count_kernel(const uint32_t *__restrict__ in,
                                                                 int64_t n, uint32_t num_tiles,
                                                                 uint32_t *__restrict__ clear_counts) {
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    uint32_t acc[32];
#pragma unroll
    for (int b = 0; b < 32; ++b) acc[b] = 0;
    for (uint32_t tile = blockIdx.x; tile < num_tiles; tile += gridDim.x) {
        const int64_t tile_start = static_cast<int64_t>(tile) * kTile;
        const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
        const bool full = tile_start + kTile <= n;
        uint32_t v[kLoads][4];
        load_chunk<VEC>(in, chunk, lane, n, full, v);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool valid = full || at + k < n;
                const uint32_t x = v[j][k];
#pragma unroll
                for (int b = 0; b < 32; ++b)
                    acc[b] += static_cast<uint32_t>(
                        __builtin_popcountll(ballot(valid && ((x >> b) & 1u) == 0u)));
            }
        }
    }
    uint32_t mine = 0;
#pragma unroll
    for (int b = 0; b < 32; ++b) mine = (lane == b) ? acc[b] : mine;
    if (lane < 32 && mine != 0)
        __hip_atomic_fetch_add(clear_counts + lane, mine, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// ================================================ unordered (atomic) kernel ---
// Comparison only: no scan, no order. VARIANT 0: each wavefront takes one
// slot range of size popcount for its whole chunk with one atomic add;
// VARIANT 1: one atomic add per survivor. *count must be zero beforehand.
template <int P, bool VEC, int VARIANT>
__global__ __launch_bounds__(kBlock) void compact_atomic_kernel(const int32_t *__restrict__ in,
                                                                int32_t *__restrict__ out,
                                                                int64_t n, int32_t pa, int32_t pb,
                                                                int32_t *__restrict__ count) {
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t tile_start = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
    const bool full = tile_start + kTile <= n;
    int32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, n, full, v);
    if constexpr (VARIANT == 0) {
        bool f[kLoads][4];
        uint32_t kb[kLoads][4];
        const uint32_t total = chunk_ranks<P>(v, chunk, lane, n, full, pa, pb, f, kb);
        uint32_t slot = 0;
        if (lane == 0 && total != 0)
            slot = static_cast<uint32_t>(__hip_atomic_fetch_add(
                count, static_cast<int32_t>(total), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        slot = uniform(slot);
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (f[j][k] && slot + kb[j][k] < n) out[slot + kb[j][k]] = v[j][k];
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t at = chunk + j * (kWave * 4) + lane * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if ((full || at + k < n) && pred_eval<P>(v[j][k], pa, pb)) {
                    const int32_t slot = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT);
                    if (slot < n) out[slot] = v[j][k];
                }
            }
        }
    }
}

// ============================================================ copy kernel ---
template <bool VEC>
__global__ __launch_bounds__(kBlock) void copy_kernel(const int32_t *__restrict__ in,
                                                      int32_t *__restrict__ out, int64_t n) {
    const int lane = lane_id();
    const int w = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t tile_start = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t chunk = tile_start + static_cast<int64_t>(w) * kChunk;
    const bool full = tile_start + kTile <= n;
    int32_t v[kLoads][4];
    load_chunk<VEC>(in, chunk, lane, n, full, v);
    store_chunk<VEC>(out, chunk, lane, n, full, v);
}

// Clears `words` 32-bit words (scratch: counters and descriptors; a kernel
// rather than a memset node).
__global__ __launch_bounds__(kBlock) void clear_kernel(uint32_t *__restrict__ p, int64_t words) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < words;
         i += static_cast<int64_t>(gridDim.x) * kBlock)
        p[i] = 0u;
}

}  // namespace ssc

// ======================================================================
// Host side: argument checks, scratch clearing, dispatch.
// ======================================================================
namespace {

using namespace ssc;

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return SSC_ERR_HIP;
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

int check_n(int64_t n) {
    if (n < 0) return SSC_ERR_ARG;
    if (n > INT32_MAX) return SSC_ERR_SIZE;
    return SSC_OK;
}

int check_scratch(const void *scratch, size_t bytes, size_t need) {
    if (scratch == nullptr || !aligned(scratch, 8) || bytes < need) return SSC_ERR_SCRATCH;
    return SSC_OK;
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

// Scratch header: word 0 the tile counter, word 1 the look-back time-out
// flag; the descriptors follow the header.
struct Scratch {
    uint32_t *counter;
    uint32_t *timed_out;
    uint64_t *desc;
};

Scratch carve(void *scratch) {
    Scratch s;
    s.counter = static_cast<uint32_t *>(scratch);
    s.timed_out = s.counter + 1;
    s.desc = reinterpret_cast<uint64_t *>(static_cast<char *>(scratch) + kHeaderBytes);
    return s;
}

size_t scratch_need(int64_t n) {
    const int64_t t = n > 0 ? tiles_for(n) : 0;
    return kHeaderBytes + static_cast<size_t>(t) * sizeof(uint64_t);
}

// ---- template dispatch on the predicate and the load width ----
template <template <int, bool> class F, class... A>
int dispatch_pred(int pred, bool vec, A... a) {
    switch (pred) {
    case 0: return vec ? F<0, true>::run(a...) : F<0, false>::run(a...);
    case 1: return vec ? F<1, true>::run(a...) : F<1, false>::run(a...);
    case 2: return vec ? F<2, true>::run(a...) : F<2, false>::run(a...);
    case 3: return vec ? F<3, true>::run(a...) : F<3, false>::run(a...);
    case 4: return vec ? F<4, true>::run(a...) : F<4, false>::run(a...);
    default: return vec ? F<5, true>::run(a...) : F<5, false>::run(a...);
    }
}

template <int P, bool VEC>
struct LaunchSelect {
    static int run(bool partition, const int32_t *in, int32_t *out, int64_t n, int32_t pa,
                   int32_t pb, Scratch sc, uint32_t tiles, int32_t *count, int32_t *ranks,
                   const int32_t *kept, hipStream_t s) {
        if (partition)
            hipLaunchKernelGGL((select_kernel<P, VEC, true>), dim3(tiles), dim3(kBlock), 0, s, in,
                               out, n, pa, pb, sc.desc, sc.counter, sc.timed_out, tiles, count,
                               ranks, kept);
        else
            hipLaunchKernelGGL((select_kernel<P, VEC, false>), dim3(tiles), dim3(kBlock), 0, s, in,
                               out, n, pa, pb, sc.desc, sc.counter, sc.timed_out, tiles, count,
                               ranks, kept);
        return launched();
    }
};

template <int P, bool VEC>
struct LaunchCount {
    static int run(const int32_t *in, int64_t n, int32_t pa, int32_t pb, uint32_t tiles,
                   int32_t *count, hipStream_t s) {
        const uint32_t grid = tiles < static_cast<uint32_t>(kReduceGrid) ? tiles : kReduceGrid;
        hipLaunchKernelGGL((count_kernel<P, VEC>), dim3(grid), dim3(kBlock), 0, s, in, n, pa, pb,
                           tiles, count);
        return launched();
    }
};

template <int P, bool VEC>
struct LaunchAtomic {
    static int run(int variant, const int32_t *in, int32_t *out, int64_t n, int32_t pa,
                   int32_t pb, uint32_t tiles, int32_t *count, hipStream_t s) {
        if (variant == 0)
            hipLaunchKernelGGL((compact_atomic_kernel<P, VEC, 0>), dim3(tiles), dim3(kBlock), 0, s,
                               in, out, n, pa, pb, count);
        else
            hipLaunchKernelGGL((compact_atomic_kernel<P, VEC, 1>), dim3(tiles), dim3(kBlock), 0, s,
                               in, out, n, pa, pb, count);
        return launched();
    }
};

#define SSC_TRY(expr)                 \
    do {                              \
        const int rc_ = (expr);       \
        if (rc_ != SSC_OK) return rc_; \
    } while (0)

template <class Op>
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
    if (overlap(scratch, scratch_need(n), in, bytes) || overlap(scratch, scratch_need(n), out, bytes) ||
        (total && overlap(scratch, scratch_need(n), total, sizeof(T))))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return total ? clear_words(total, 1, s) : SSC_OK;
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    SSC_TRY(clear_words(scratch, static_cast<int64_t>(scratch_need(n) / 4), s));
    const Scratch sc = carve(scratch);
    if (aligned(in, 16) && aligned(out, 16))
        hipLaunchKernelGGL((scan_kernel<Op, true>), dim3(tiles), dim3(kBlock), 0, s, in, out, n,
                           sc.desc, sc.counter, sc.timed_out, tiles, total);
    else
        hipLaunchKernelGGL((scan_kernel<Op, false>), dim3(tiles), dim3(kBlock), 0, s, in, out, n,
                           sc.desc, sc.counter, sc.timed_out, tiles, total);
    return launched();
}

}  // namespace

// ======================================================================
// C ABI
// ======================================================================
extern "C" {

int64_t ssc_tile_elems(void) { return kTile; }

size_t ssc_scratch_bytes(int64_t n) { return scratch_need(n < 0 ? 0 : n); }

size_t ssc_radix_sort_scratch_bytes(int64_t n) {
    const int64_t t = n > 0 ? tiles_for(n) : 0;
    return kRadixHeaderBytes + 32 * static_cast<size_t>(t) * sizeof(uint64_t);
}

int ssc_exclusive_scan_i32(const int32_t *in, int32_t *out, int64_t n, int32_t *total,
                           void *scratch, size_t scratch_bytes, void *stream) {
    return scan_impl<SumU32>(reinterpret_cast<const uint32_t *>(in), reinterpret_cast<uint32_t *>(out),
                             n, reinterpret_cast<uint32_t *>(total), scratch, scratch_bytes,
                             static_cast<hipStream_t>(stream));
}

int ssc_exclusive_scan_f32(const float *in, float *out, int64_t n, float *total, void *scratch,
                           size_t scratch_bytes, void *stream) {
    return scan_impl<SumF32>(in, out, n, total, scratch, scratch_bytes,
                             static_cast<hipStream_t>(stream));
}

int ssc_compact_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa, int32_t pb,
                    int32_t *count, int32_t *ranks, void *scratch, size_t scratch_bytes,
                    void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || out == nullptr))) return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(count, 4) || (ranks && !aligned(ranks, 4)))
        return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    const size_t need = scratch_need(n);
    if (overlap(in, bytes, out, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, out, bytes) ||
        (ranks && (overlap(ranks, bytes, in, bytes) || overlap(ranks, bytes, out, bytes) ||
                   overlap(ranks, bytes, count, 4))))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, need));
    if (overlap(scratch, need, in, bytes) || overlap(scratch, need, out, bytes) ||
        overlap(scratch, need, count, 4) || (ranks && overlap(scratch, need, ranks, bytes)))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return clear_words(count, 1, s);
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    SSC_TRY(clear_words(scratch, static_cast<int64_t>(need / 4), s));
    const bool vec = aligned(in, 16) && (ranks == nullptr || aligned(ranks, 16));
    return dispatch_pred<LaunchSelect>(pred, vec, false, in, out, n, pa, pb, carve(scratch), tiles,
                                       count, ranks, static_cast<const int32_t *>(nullptr), s);
}

int ssc_partition_i32(const int32_t *in, int32_t *out, int64_t n, int pred, int32_t pa, int32_t pb,
                      int32_t *count, void *scratch, size_t scratch_bytes, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && (in == nullptr || out == nullptr))) return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(out, 4) || !aligned(count, 4)) return SSC_ERR_ARG;
    const size_t bytes = static_cast<size_t>(n) * 4;
    const size_t need = scratch_need(n);
    if (overlap(in, bytes, out, bytes) || overlap(count, 4, in, bytes) ||
        overlap(count, 4, out, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_scratch(scratch, scratch_bytes, need));
    if (overlap(scratch, need, in, bytes) || overlap(scratch, need, out, bytes) ||
        overlap(scratch, need, count, 4))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    SSC_TRY(clear_words(count, 1, s));
    if (n == 0) return SSC_OK;
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    SSC_TRY(clear_words(scratch, static_cast<int64_t>(need / 4), s));
    const bool vec = aligned(in, 16);
    SSC_TRY(dispatch_pred<LaunchCount>(pred, vec, in, n, pa, pb, tiles, count, s));
    return dispatch_pred<LaunchSelect>(pred, vec, true, in, out, n, pa, pb, carve(scratch), tiles,
                                       static_cast<int32_t *>(nullptr),
                                       static_cast<int32_t *>(nullptr),
                                       static_cast<const int32_t *>(count), s);
}

int ssc_count_if_i32(const int32_t *in, int64_t n, int pred, int32_t pa, int32_t pb,
                     int32_t *count, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    SSC_TRY(check_n(n));
    if (count == nullptr || (n > 0 && in == nullptr)) return SSC_ERR_ARG;
    SSC_TRY(check_pred(pred, pa, pb));
    if (!aligned(in, 4) || !aligned(count, 4)) return SSC_ERR_ARG;
    if (overlap(count, 4, in, static_cast<size_t>(n) * 4)) return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    SSC_TRY(clear_words(count, 1, s));
    if (n == 0) return SSC_OK;
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    return dispatch_pred<LaunchCount>(pred, aligned(in, 16), in, n, pa, pb, tiles, count, s);
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
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    return dispatch_pred<LaunchAtomic>(pred, aligned(in, 16), variant, in, out, n, pa, pb, tiles,
                                       count, s);
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
    const size_t need = ssc_radix_sort_scratch_bytes(n);
    SSC_TRY(check_scratch(scratch, scratch_bytes, need));
    if (overlap(scratch, need, in, bytes) || overlap(scratch, need, out, bytes) ||
        overlap(scratch, need, tmp, bytes))
        return SSC_ERR_ALIAS;
    SSC_TRY(check_device());
    if (n == 0) return SSC_OK;
    const int64_t tiles64 = tiles_for(n);
    const uint32_t tiles = static_cast<uint32_t>(tiles64);
    SSC_TRY(clear_words(scratch, static_cast<int64_t>(need / 4), s));
    // Header: 32 tile counters (one per pass), 32 bit-clear counts, then the
    // look-back time-out flag; 32 descriptor arrays follow.
    uint32_t *counters = static_cast<uint32_t *>(scratch);
    uint32_t *clear_counts = counters + 32;
    uint32_t *timed_out = counters + 64;
    uint64_t *desc0 =
        reinterpret_cast<uint64_t *>(static_cast<char *>(scratch) + kRadixHeaderBytes);
    const bool vec = aligned(in, 16) && aligned(out, 16) && aligned(tmp, 16);
    {
        const uint32_t grid = tiles < static_cast<uint32_t>(kReduceGrid) ? tiles : kReduceGrid;
        if (vec)
            hipLaunchKernelGGL((bit_clear_count_kernel<true>), dim3(grid), dim3(kBlock), 0, s, in,
                               n, tiles, clear_counts);
        else
            hipLaunchKernelGGL((bit_clear_count_kernel<false>), dim3(grid), dim3(kBlock), 0, s, in,
                               n, tiles, clear_counts);
        SSC_TRY(launched());
    }
    const uint32_t *src = in;
    for (int b = 0; b < 32; ++b) {
        uint32_t *dst = (b % 2 == 0) ? tmp : out;  // pass 31 lands in out
        Scratch sc;
        sc.counter = counters + b;
        sc.timed_out = timed_out;
        sc.desc = desc0 + static_cast<size_t>(b) * tiles64;
        const int32_t *kept = reinterpret_cast<const int32_t *>(clear_counts + b);
        if (vec)
            SSC_TRY((LaunchSelect<4, true>::run(true, reinterpret_cast<const int32_t *>(src),
                                                reinterpret_cast<int32_t *>(dst), n, b, 0, sc,
                                                tiles, nullptr, nullptr, kept, s)));
        else
            SSC_TRY((LaunchSelect<4, false>::run(true, reinterpret_cast<const int32_t *>(src),
                                                 reinterpret_cast<int32_t *>(dst), n, b, 0, sc,
                                                 tiles, nullptr, nullptr, kept, s)));
        src = dst;
    }
    return SSC_OK;
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
    const uint32_t tiles = static_cast<uint32_t>(tiles_for(n));
    if (aligned(in, 16) && aligned(out, 16))
        hipLaunchKernelGGL((copy_kernel<true>), dim3(tiles), dim3(kBlock), 0, s, in, out, n);
    else
        hipLaunchKernelGGL((copy_kernel<false>), dim3(tiles), dim3(kBlock), 0, s, in, out, n);
    return launched();
}

const char *ssc_status_str(int status) {
    switch (status) {
    case SSC_OK: return "ok";
    case SSC_ERR_ARG: return "invalid argument";
    case SSC_ERR_SIZE: return "n exceeds INT32_MAX";
    case SSC_ERR_ALIAS: return "buffers overlap";
    case SSC_ERR_SCRATCH: return "scratch too small or misaligned";
    case SSC_ERR_HIP: return "HIP error";
    case SSC_ERR_DEVICE: return "device is not gfx950 with 64-wide wavefronts";
    default: return "unknown status";
    }
}

int ssc_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
