// COO -> CSR by key: a stable least-significant-digit radix sort of (key, COO index,
// other endpoint).
//
// A build takes ceil(bits / 7) passes over the key bits (three for n <= 2^21), each sorting
// by one digit of at most 7 bits.  A pass is stable by construction: each wavefront of a
// 4096-item tile ranks its own contiguous run of items in their original order (64 at a
// time, the lanes with equal digits found through a per-digit lane mask in LDS, a per-digit
// running count in LDS carrying over from one 64-item round to the next), the wavefronts'
// runs are placed in wavefront order (per-digit counts of each wavefront, scanned in LDS),
// and tiles are ordered by each digit's exclusive scan of its per-tile counts over the
// tiles, offset by the totals of the smaller digits.  The result therefore equals a stable
// sort, independent of scheduling: within a row the COO indices ascend, bit-exact across
// runs and devices.  The other endpoint travels with each item, so the last pass writes
// col directly.  Each tile is staged in LDS in digit order before it is written, so the
// scatter writes contiguous runs.  row_ptr comes from the segment boundaries of the sorted
// keys; no atomics decide any position.
#include "common.hpp"

namespace gga {

namespace {

constexpr int kMaxDigitBits = 7;
constexpr int kMaxBins = 1 << kMaxDigitBits;
constexpr int kRsWaves = 8;
constexpr int kRsThreads = 64 * kRsWaves;
constexpr int kRsRounds = 8;                     // 64-item rounds per wavefront
constexpr int kRsWaveItems = 64 * kRsRounds;     // a wavefront's contiguous run of a tile
constexpr int kRsTile = kRsThreads * kRsRounds;  // 4096 edges per tile
// digits per thread in the tile scan: whole words of two 16-bit counters
constexpr int kDigitsPerThread = kMaxBins / kRsThreads < 2 ? 2 : kMaxBins / kRsThreads;

__global__ void count_bad(const int32_t* __restrict__ a, const int32_t* __restrict__ b, int64_t e, int32_t n,
                          int32_t* __restrict__ bad) {
    int local = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < e; i += (int64_t)gridDim.x * blockDim.x)
        local += ((uint32_t)a[i] >= (uint32_t)n) + ((uint32_t)b[i] >= (uint32_t)n);
    if (local) atomicAdd(bad, local);
}

__device__ __forceinline__ uint32_t digit_of(int32_t key, int shift, uint32_t mask) {
    return ((uint32_t)key >> shift) & mask;
}

// Lanes of the wavefront whose item is valid and has digit d (as this lane's), for a valid
// lane (the valid lanes are a prefix of the wavefront).  When every valid lane has lane 0's
// digit (a round inside a long row of one key) they are the valid lanes.  Otherwise `mask`,
// the wavefront's table of one 64-bit lane mask per digit, all zero on entry and on return,
// finds them: every valid lane ORs its bit into its digit's mask, reads the mask back and
// clears it.  The three are single instructions of the whole wavefront, and a wavefront's LDS
// operations complete in issue order, so each read sees the bits of every lane of the round
// and each clear comes after every read of the round.
__device__ __forceinline__ uint64_t same_digit_lanes(uint64_t* mask, uint32_t d, bool valid, uint64_t bit) {
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
    const uint64_t vm = __ballot(valid);
    if (__all(!valid || d == d0)) return valid ? vm : 0ull;
    uint64_t peers = 0;
    if (valid) {
        __hip_atomic_fetch_or(mask + d, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        peers = __hip_atomic_load(mask + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        __hip_atomic_store(mask + d, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
    return peers;
}

// Workgroups go to the eight XCDs in turn (workgroup b to XCD b % 8); the tile of workgroup
// b is chosen so that each XCD takes one contiguous range of tiles, in order.  Runs of one
// digit from neighbouring tiles are neighbours in the output, and so are neighbouring tiles'
// entries of a digit's histogram row: the cache line shared by two tiles' writes is then
// written by one XCD's L2, close in time, and leaves it whole rather than as partial lines.
// (Any mapping is correct: this one is a bijection of [0, nblocks).)
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t nblocks) {
    const int64_t x = b % kXcds, k = b / kXcds, q = nblocks / kXcds, r = nblocks % kXcds;
    return x * q + (x < r ? x : r) + k;
}

// Per-tile digit counts: hist[d * nblocks + tile].  Each wavefront counts into its own
// histogram (fewer conflicting LDS additions), and the wavefronts' histograms are summed at
// the end.  A whole tile of 16-byte aligned keys is read as 16-byte vectors, a lane taking
// consecutive keys; a wavefront whose keys all share one digit adds once.
__global__ __launch_bounds__(kRsThreads) void radix_upsweep(const int32_t* __restrict__ keys, int64_t e, int shift,
                                                            int bits, int32_t* __restrict__ hist, int64_t nblocks) {
    __shared__ int cnt[kRsWaves][kMaxBins];
    const int bins = 1 << bits;
    const uint32_t mask = (uint32_t)bins - 1u;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // (each wavefront clears and fills only its own histogram before the barrier)
    for (int d = lane; d < bins; d += 64) cnt[wave][d] = 0;
    const int64_t tile = xcd_tile(blockIdx.x, nblocks);
    const int64_t base = tile * kRsTile;
    static_assert(kRsRounds % 4 == 0, "whole 16-byte vectors per thread");
    if (base + kRsTile <= e && (reinterpret_cast<uintptr_t>(keys) & 15) == 0) {
        // each lane counts kRsRounds consecutive keys: runs of one digit (long rows of one
        // key, or keys sorted by earlier passes) become one addition each
        const int4* kv = reinterpret_cast<const int4*>(keys + base) + tid * (kRsRounds / 4);
        uint32_t d[kRsRounds];
#pragma unroll
        for (int r = 0; r < kRsRounds / 4; r++) {
            const int4 k = kv[r];
            d[4 * r] = digit_of(k.x, shift, mask);
            d[4 * r + 1] = digit_of(k.y, shift, mask);
            d[4 * r + 2] = digit_of(k.z, shift, mask);
            d[4 * r + 3] = digit_of(k.w, shift, mask);
        }
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(d[0]);
        bool same = true;
#pragma unroll
        for (int r = 0; r < kRsRounds; r++) same = same && d[r] == d0;
        if (__all(same)) {
            if (lane == 0) atomicAdd(&cnt[wave][d0], 64 * kRsRounds);
        } else {
            uint32_t cur = d[0];
            int c = 1;
#pragma unroll
            for (int r = 1; r < kRsRounds; r++) {
                if (d[r] == cur) {
                    c++;
                } else {
                    atomicAdd(&cnt[wave][cur], c);
                    cur = d[r];
                    c = 1;
                }
            }
            atomicAdd(&cnt[wave][cur], c);
        }
    } else {
        int32_t k[kRsRounds];
#pragma unroll
        for (int r = 0; r < kRsRounds; r++) {
            const int64_t i = base + r * kRsThreads + tid;
            k[r] = i < e ? keys[i] : 0;
        }
#pragma unroll
        for (int r = 0; r < kRsRounds; r++) {
            const int64_t i = base + r * kRsThreads + tid;
            if (i < e) atomicAdd(&cnt[wave][digit_of(k[r], shift, mask)], 1);
        }
    }
    __syncthreads();
    for (int d = tid; d < bins; d += kRsThreads) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kRsWaves; w++) c += cnt[w][d];
        hist[(int64_t)d * nblocks + tile] = c;
    }
}

// Each digit's row of per-tile counts hist[d * nblocks + t] becomes its exclusive scan over
// the tiles, in place, and totals[d] the digit's count.  One workgroup per digit; a thread
// takes kDsItems consecutive tiles of each kDsThreads * kDsItems (6144: one round for up to
// 25M edges, where a round's barriers and latency are most of the kernel's time).
constexpr int kDsThreads = 1024;
constexpr int kDsItems = 6;

__global__ __launch_bounds__(kDsThreads) void digit_rows_scan(int32_t* __restrict__ hist, int64_t nblocks,
                                                              int32_t* __restrict__ totals) {
    __shared__ int32_t wtot[kDsThreads / 64];
    int32_t* row = hist + (int64_t)blockIdx.x * nblocks;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t carry = 0;
    for (int64_t base = 0; base < nblocks; base += (int64_t)kDsThreads * kDsItems) {
        int32_t v[kDsItems];
        int32_t sum = 0;
#pragma unroll
        for (int j = 0; j < kDsItems; j++) {
            const int64_t i = base + (int64_t)tid * kDsItems + j;
            v[j] = i < nblocks ? row[i] : 0;
            sum += v[j];
        }
        int32_t x = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wtot[wave] = x;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kDsThreads / 64; w++) {
            const int32_t t = wtot[w];
            before += w < wave ? t : 0;
            total += t;
        }
        __syncthreads();  // (wtot is rewritten by the next chunk)
        int32_t run = carry + before + x - sum;
#pragma unroll
        for (int j = 0; j < kDsItems; j++) {
            const int64_t i = base + (int64_t)tid * kDsItems + j;
            if (i < nblocks) row[i] = run;
            run += v[j];
        }
        carry += total;
    }
    if (tid == 0) totals[blockIdx.x] = carry;
}

// row_ptr[v] = p for the rows v in (prev, key], clamped to [0, n]: position p holds the first
// item of those rows when the keys are sorted and the item before it has key prev.  Every
// write stays in bounds, whatever the keys.
__device__ __forceinline__ void fill_rows(int32_t* row_ptr, int32_t n, int64_t prev, int64_t key, int64_t p) {
    const int64_t lo = prev + 1 < 0 ? 0 : prev + 1;
    const int64_t hi = key < n ? key : n;
    for (int64_t v = lo; v <= hi; v++) row_ptr[v] = (int32_t)p;
}

// A wavefront's items of one tile, in order: round r, lane l holds item wbase + 64 r + l.
struct TileItems {
    int32_t key[kRsRounds], val[kRsRounds], oth[kRsRounds];
};

struct RadixArgs {
    const int32_t* keys_in;
    const int32_t* vals_in;  // null in the first pass: the values are the COO indices
    const int32_t* oth_in;
    int32_t* keys_out;  // may be null (keys not needed after this pass)
    int32_t* vals_out;
    int32_t* oth_out;
    const int32_t* offsets;  // per digit, the exclusive scan of its per-tile counts over the tiles
    const int32_t* totals;   // per digit, its count over all tiles
    int64_t e, nblocks;
    int shift, bits;
    // last pass only (null otherwise): row_ptr is written from the tile's sorted keys.  Each
    // tile's run of each digit leaves its first key and global start in run_key / run_pos
    // ([digit * nblocks + tile]; start -1 for an empty run), and its last key in run_lkey;
    // row_ptr_gaps fills the rows between runs.
    int32_t* row_ptr;
    int32_t* run_key;
    int32_t* run_pos;
    int32_t* run_lkey;  // the key of each run's last item
    int32_t n;
};

struct RadixSmem {
    // a wavefront's 16-bit per-digit counts, then its next tile position per digit; digit d
    // sits in half d & 1 of word d / 2 (positions stay below 2^16, so halves never carry)
    uint32_t wpos[kRsWaves][kMaxBins / 2];
    uint16_t tdo[kMaxBins];   // tile-local start of each digit
    uint16_t tcnt[kMaxBins];  // the tile's count of each digit
    int32_t gbase[kMaxBins];  // global start of each digit's run of this tile
    int32_t wtot[kRsWaves];
    int32_t wtot_all[kRsWaves];
    union {
        // while the wavefronts rank their items: each one's lane mask per digit
        uint64_t lanes[kRsWaves][kMaxBins];
        // then the tile in (digit, original order)
        struct {
            int32_t skey[kRsTile];
            int32_t sval[kRsTile];
            int32_t soth[kRsTile];
        };
    };
};

__device__ __forceinline__ int tile_size(const RadixArgs& a, int64_t tile) {
    const int64_t rest = a.e - tile * kRsTile;
    return (int)(rest < kRsTile ? rest : kRsTile);
}

template <bool FIRST>
__device__ __forceinline__ void load_tile(const RadixArgs& a, int64_t tile, TileItems& it) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t base = tile * kRsTile;
    const int tile_n = tile_size(a, tile);
#pragma unroll
    for (int r = 0; r < kRsRounds; r++) {
        const int li = wave * kRsWaveItems + r * 64 + lane;
        const bool valid = li < tile_n;
        it.key[r] = valid ? a.keys_in[base + li] : 0;
        it.oth[r] = valid ? a.oth_in[base + li] : 0;
        if constexpr (FIRST)
            it.val[r] = (int32_t)(base + li);
        else
            it.val[r] = valid ? a.vals_in[base + li] : 0;
    }
}

// Sorts one tile's items stably by the digit (key >> shift) & (2^bits - 1) and writes them
// to their places.
__device__ __forceinline__ void sort_tile(const RadixArgs& a, int64_t tile, const TileItems& it, RadixSmem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bits = a.bits, shift = a.shift;
    const int bins = 1 << bits;
    const int words = (bins + 1) / 2;
    const uint32_t mask = (uint32_t)bins - 1u;
    const int64_t base = tile * kRsTile;
    const int tile_n = tile_size(a, tile);
    const int wbase = wave * kRsWaveItems;

    // the starts of this tile's runs of the thread's digits among the digits' runs of all
    // tiles, and the digits' totals (used after the ranking; loaded first, so their latency
    // passes under it)
    int32_t gb[kDigitsPerThread], dt[kDigitsPerThread];
#pragma unroll
    for (int j = 0; j < kDigitsPerThread; j++) {
        const int d = tid * kDigitsPerThread + j;
        gb[j] = d < bins ? a.offsets[(int64_t)d * a.nblocks + tile] : 0;
        dt[j] = d < bins ? a.totals[d] : 0;
    }
    for (int i = tid; i < kRsWaves * (kMaxBins / 2); i += kRsThreads) {
        const int w = i / (kMaxBins / 2), x = i % (kMaxBins / 2);
        if (x < words) sm.wpos[w][x] = 0;
    }
    // (each wavefront clears its own lane masks, so they need no barrier before its ranking)
    for (int x = lane; x < bins; x += 64) sm.lanes[wave][x] = 0;
    __syncthreads();

    // each wavefront ranks its items among the equal digits of their 64-item round, and the
    // first lane of each group adds the group's size to the wavefront's count of the digit
    // (additions commute: no ordering needed).  rl[r]: rank in the group | group size << 16.
    uint32_t rl[kRsRounds];
    {
        const uint64_t bit = 1ull << lane;
#pragma unroll
        for (int r = 0; r < kRsRounds; r++) {
            const bool valid = wbase + r * 64 + lane < tile_n;
            const uint32_t d = digit_of(it.key[r], shift, mask);
            const uint64_t peers = same_digit_lanes(sm.lanes[wave], d, valid, bit);
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
            const uint32_t size = (uint32_t)__popcll(peers);
            rl[r] = rank | (size << 16);
            // (materialise the packed word here, so the 64-bit masks do not stay live)
            asm volatile("" : "+v"(rl[r]));
            if (valid && rank == 0) atomicAdd(&sm.wpos[wave][d >> 1], size << (16 * (d & 1)));
        }
    }
    __syncthreads();

    // tile-local digit starts (scan over digits), each wavefront's start per digit (in
    // wavefront order), and the global start of each digit's run of this tile.  A thread
    // owns kDigitsPerThread consecutive digits, i.e. whole words of wpos.
    {
        int c[kDigitsPerThread];
        int tot = 0, tot_all = 0;
#pragma unroll
        for (int j = 0; j < kDigitsPerThread; j++) {
            const int d = tid * kDigitsPerThread + j;
            c[j] = 0;
            if (d < bins)
                for (int w = 0; w < kRsWaves; w++) c[j] += (sm.wpos[w][d >> 1] >> (16 * (d & 1))) & 0xffffu;
            tot += c[j];
            tot_all += dt[j];
        }
        int x = tot, xa = tot_all;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64), ya = __shfl_up(xa, off, 64);
            if (lane >= off) {
                x += y;
                xa += ya;
            }
        }
        if (lane == 63) {
            sm.wtot[wave] = x;
            sm.wtot_all[wave] = xa;
        }
        __syncthreads();
        int run = x - tot, run_all = xa - tot_all;  // run_all: the first position of the thread's first digit
        for (int w = 0; w < wave; w++) {
            run += sm.wtot[w];
            run_all += sm.wtot_all[w];
        }
#pragma unroll
        for (int m = 0; m < kDigitsPerThread / 2; m++) {
            const int d0 = tid * kDigitsPerThread + 2 * m;
            if (d0 < bins) {
                uint32_t s0 = (uint32_t)run, s1 = (uint32_t)(run + c[2 * m]);
                sm.tdo[d0] = (uint16_t)s0;
                sm.tcnt[d0] = (uint16_t)c[2 * m];
                sm.gbase[d0] = run_all + gb[2 * m];
                if (a.row_ptr && c[2 * m] == 0) a.run_pos[(int64_t)d0 * a.nblocks + tile] = -1;
                if (d0 + 1 < bins) {
                    sm.tdo[d0 + 1] = (uint16_t)s1;
                    sm.tcnt[d0 + 1] = (uint16_t)c[2 * m + 1];
                    sm.gbase[d0 + 1] = run_all + dt[2 * m] + gb[2 * m + 1];
                    if (a.row_ptr && c[2 * m + 1] == 0) a.run_pos[(int64_t)(d0 + 1) * a.nblocks + tile] = -1;
                }
                for (int w = 0; w < kRsWaves; w++) {
                    const uint32_t cw = sm.wpos[w][d0 >> 1];
                    sm.wpos[w][d0 >> 1] = s0 | (s1 << 16);
                    s0 += cw & 0xffffu;
                    s1 += cw >> 16;
                }
            }
            run += c[2 * m] + c[2 * m + 1];
            run_all += dt[2 * m] + dt[2 * m + 1];
        }
    }
    __syncthreads();

    // each wavefront places its items in order.  Per round every item reads its digit's next
    // position and the first lane of each group of equal digits then adds the group's size;
    // a wavefront's LDS operations complete in issue order, so the reads see the earlier
    // rounds' additions and not this round's, and every group lands after the earlier
    // rounds' items of its digit.  (The staging overlays the lane masks, whose last use is
    // before the barrier above.)
#pragma unroll
    for (int r = 0; r < kRsRounds; r++) {
        const bool valid = wbase + r * 64 + lane < tile_n;
        if (valid) {
            const uint32_t d = digit_of(it.key[r], shift, mask);
            uint32_t* wp = &sm.wpos[wave][d >> 1];
            const uint32_t w0 = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
            const uint32_t rank = rl[r] & 0xffffu;
            if (rank == 0)
                __hip_atomic_fetch_add(wp, (rl[r] >> 16) << (16 * (d & 1)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WAVEFRONT);
            const int pos = (int)((w0 >> (16 * (d & 1))) & 0xffffu) + (int)rank;
            sm.skey[pos] = it.key[r];
            sm.sval[pos] = it.val[r];
            sm.soth[pos] = it.oth[r];
        }
    }
    __syncthreads();

    // the tile now sits in LDS in (digit, original order); write each digit's run contiguously
    for (int li = tid; li < tile_n; li += kRsThreads) {
        const int32_t k = sm.skey[li];
        const uint32_t d = digit_of(k, shift, mask);
        const int first = sm.tdo[d], last = first + (int)sm.tcnt[d] - 1;
        const int64_t pos = (int64_t)sm.gbase[d] + (li - first);
        a.vals_out[pos] = sm.sval[li];
        a.oth_out[pos] = sm.soth[li];
        if (!a.row_ptr) {
            if (a.keys_out) a.keys_out[pos] = k;
            continue;
        }
        // after the last pass the keys are sorted: within a run the rows between the previous
        // key and this one start here; a run's first item leaves that to row_ptr_gaps
        if (li == first) {
            a.run_key[(int64_t)d * a.nblocks + tile] = k;
            a.run_pos[(int64_t)d * a.nblocks + tile] = (int32_t)pos;
        } else {
            fill_rows(a.row_ptr, a.n, sm.skey[li - 1], k, pos);
        }
        if (li == last) {
            a.run_lkey[(int64_t)d * a.nblocks + tile] = k;
            if (pos == a.e - 1) fill_rows(a.row_ptr, a.n, k, a.n, a.e);  // the rows after the largest key
        }
    }
    (void)base;
}

// One pass: one workgroup per tile.
template <bool FIRST>
__global__ __launch_bounds__(kRsThreads) void radix_downsweep(RadixArgs a) {
    __shared__ RadixSmem sm;
    TileItems x;
    const int64_t tile = xcd_tile(blockIdx.x, a.nblocks);
    load_tile<FIRST>(a, tile, x);
    sort_tile(a, tile, x, sm);
}

// row_ptr_gaps: the rows between a tile run's first key and the key of the item before it
// start at the run's first position p.  That item is the last of the closest earlier
// non-empty run in digit-major order (the order of the output).  A thread takes kGapRuns
// consecutive runs, their loads issued together: within the group that run is the previous
// non-empty one of the group, and only the group's first non-empty run looks further back,
// stepping back over empty runs or, past kGapSteps of them, by a binary search of the runs'
// starts (dbase[d] + offsets[d][t], non-decreasing) for the run that holds position p - 1.
constexpr int kGapSteps = 32;
constexpr int kGapRuns = 4;

__global__ __launch_bounds__(256) void row_ptr_gaps(const int32_t* __restrict__ run_key,
                                                    const int32_t* __restrict__ run_pos,
                                                    const int32_t* __restrict__ run_lkey,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ totals, int bits, int64_t nblocks,
                                                    int32_t n, int32_t* __restrict__ row_ptr) {
    __shared__ int32_t dbase[kMaxBins];
    const int bins = 1 << bits;
    if (threadIdx.x < 64) {  // exclusive scan of the digits' totals, two digits per lane
        const int lane = threadIdx.x;
        const int32_t t0 = 2 * lane < bins ? totals[2 * lane] : 0, t1 = 2 * lane + 1 < bins ? totals[2 * lane + 1] : 0;
        int32_t x = t0 + t1;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const int32_t ex = x - t0 - t1;
        if (2 * lane < bins) dbase[2 * lane] = ex;
        if (2 * lane + 1 < bins) dbase[2 * lane + 1] = ex + t0;
    }
    __syncthreads();
    const int64_t runs = (int64_t)bins * nblocks;
    const int64_t groups = (runs + kGapRuns - 1) / kGapRuns;
    for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < groups;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i0 = gi * kGapRuns;
        int32_t pos[kGapRuns], key[kGapRuns], lkey[kGapRuns];
#pragma unroll
        for (int r = 0; r < kGapRuns; r++) {  // (an empty run's keys are never used)
            const bool in = i0 + r < runs;
            pos[r] = in ? run_pos[i0 + r] : -1;
            key[r] = in ? run_key[i0 + r] : 0;
            lkey[r] = in ? run_lkey[i0 + r] : 0;
        }
        int first = kGapRuns;
#pragma unroll
        for (int r = kGapRuns - 1; r >= 0; r--)
            if (pos[r] >= 0) first = r;
        if (first == kGapRuns) continue;
        int64_t prev = -1;
        const int32_t p = pos[first];
        if (p > 0) {
            const int64_t i = i0 + first;
            int64_t j = i0 - 1;  // the runs i0 .. i - 1 are empty
            for (int step = 0; step < kGapSteps && j >= 0 && run_pos[j] < 0; step++) j--;
            if (j < 0 || run_pos[j] < 0) {
                // the largest j < i whose run starts at or before p - 1 (run 0 starts at 0)
                int64_t lo = 0, hi = i - 1;
                while (lo < hi) {
                    const int64_t mid = (lo + hi + 1) / 2;
                    if ((int64_t)dbase[mid / nblocks] + offsets[mid] <= (int64_t)p - 1)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                j = lo;
            }
            prev = run_lkey[j];
        }
#pragma unroll
        for (int r = 0; r < kGapRuns; r++) {
            if (r < first || pos[r] < 0) continue;
            fill_rows(row_ptr, n, prev, key[r], pos[r]);
            prev = lkey[r];
        }
    }
}

// Packs per-graph local COO ids into the block-diagonal list over the packed node axis.
// Entry i belongs to the graph b with edge_ptr[b] <= i < edge_ptr[b+1] (binary search).
__global__ void batch_edges_kernel(int32_t batch, const int32_t* __restrict__ node_ptr,
                                   const int32_t* __restrict__ edge_ptr, int64_t e, const int32_t* __restrict__ sl,
                                   const int32_t* __restrict__ dl, int32_t* __restrict__ src, int32_t* __restrict__ dst,
                                   int32_t* __restrict__ bad) {
    int local = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < e; i += (int64_t)gridDim.x * blockDim.x) {
        int32_t lo = 0, hi = batch + 1;  // first index with edge_ptr > i
        while (lo < hi) {
            const int32_t mid = (lo + hi) >> 1;
            if ((int64_t)edge_ptr[mid] <= i)
                lo = mid + 1;
            else
                hi = mid;
        }
        const int32_t b = lo - 1;
        int32_t s = -1, d = -1;
        if (b >= 0 && b < batch) {
            const int32_t base = node_ptr[b], nb = node_ptr[b + 1] - base;
            const int32_t a = sl[i], c = dl[i];
            if (a >= 0 && a < nb) s = a + base;
            if (c >= 0 && c < nb) d = c + base;
        }
        src[i] = s;
        dst[i] = d;
        local += (s < 0) + (d < 0);
    }
    if (local) atomicAdd(bad, local);
}

// Relation-typed edges: a launch covers up to kRelSegs consecutive host-side segments,
// passed by value; edge i takes the relation of the last segment starting at or before i
// (segments are contiguous and ordered, so that is the one holding i).
constexpr int kRelSegs = 32;

struct RelSegs {
    int32_t rel[kRelSegs];
    int32_t start[kRelSegs];
    int32_t count;
};

__global__ void relation_sources_kernel(int32_t n, int32_t n_rel, int64_t lo, int64_t hi, RelSegs sg,
                                        const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                        int32_t* __restrict__ out, int32_t* __restrict__ bad) {
    int local = 0;
    for (int64_t i = lo + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < hi;
         i += (int64_t)gridDim.x * blockDim.x) {
        int32_t r = sg.rel[0];
        for (int k = 1; k < sg.count; k++)
            if ((int64_t)sg.start[k] <= i) r = sg.rel[k];
        const int32_t u = src[i];
        const bool ok = (uint32_t)u < (uint32_t)n;
        out[i] = ok ? u * n_rel + r : -1;
        local += !ok + ((uint32_t)dst[i] >= (uint32_t)n);
    }
    if (local) atomicAdd(bad, local);
}

int key_bits(int32_t n) {
    if (n <= 1) return 0;
    uint32_t m = (uint32_t)(n - 1);
    return 32 - __builtin_clz(m);
}

// Digit width of each pass: the key bits split into ceil(bits / 8) passes of equal width
// (the last one narrower when they do not divide).
struct Passes {
    int count, width;
};

Passes passes_for(int32_t n) {
    const int bits = key_bits(n);
    Passes p;
    p.count = bits == 0 ? 1 : (bits + kMaxDigitBits - 1) / kMaxDigitBits;
    p.width = bits == 0 ? 0 : (bits + p.count - 1) / p.count;
    return p;
}

struct CsrWs {
    int32_t* hist;
    int32_t* totals;
    int32_t* run_key;
    int32_t* run_pos;
    int32_t* run_lkey;
    int32_t* keys_tmp[2];
    int32_t* vals_tmp;
    int32_t* oth_tmp;
    size_t bytes;
};

CsrWs carve(void* ws, int32_t n, int64_t e) {
    Carver c(ws);
    CsrWs w;
    const int64_t nblocks = (e + kRsTile - 1) / kRsTile;
    const int64_t hist_n = ((int64_t)1 << passes_for(n).width) * nblocks;
    w.hist = c.take<int32_t>((size_t)hist_n);
    w.totals = c.take<int32_t>((size_t)kMaxBins);
    w.run_key = c.take<int32_t>((size_t)hist_n);
    w.run_pos = c.take<int32_t>((size_t)hist_n);
    w.run_lkey = c.take<int32_t>((size_t)hist_n);
    w.keys_tmp[0] = c.take<int32_t>((size_t)e);
    w.keys_tmp[1] = c.take<int32_t>((size_t)e);
    w.vals_tmp = c.take<int32_t>((size_t)e);
    w.oth_tmp = c.take<int32_t>((size_t)e);
    w.bytes = c.bytes();
    return w;
}

int grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    if (b < 1) b = 1;
    if (b > 16384) b = 16384;
    return (int)b;
}

}  // namespace

}  // namespace gga

using namespace gga;

extern "C" size_t gga_coo_to_csr_workspace(int32_t n, int64_t e) {
    if (n < 0 || e < 0 || e >= (int64_t)INT32_MAX) return 0;
    return carve(nullptr, n, e).bytes;
}

extern "C" int gga_validate_coo(int32_t n, int64_t e, const int32_t* src, const int32_t* dst, int32_t* d_bad,
                                void* stream) {
    if (n < 0 || e < 0) return GGA_EINVAL;
    if (!d_bad || (e > 0 && (!src || !dst))) return GGA_EINVAL;
    hipStream_t s = as_stream(stream);
    fill_i32(d_bad, 1, 0, s);
    if (e > 0) count_bad<<<grid_for(e), 256, 0, s>>>(src, dst, e, n, d_bad);
    return launch_status();
}

extern "C" int gga_coo_to_csr(int32_t n, int64_t e, const int32_t* key, const int32_t* other, int32_t* row_ptr,
                              int32_t* col, int32_t* eid, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || e < 0) return GGA_EINVAL;
    if (e >= (int64_t)INT32_MAX) return GGA_ERANGE;
    if (!row_ptr) return GGA_EINVAL;
    if (e > 0 && (!key || !other || !col || !eid)) return GGA_EINVAL;
    CsrWs w = carve(nullptr, n, e);
    if (ws_bytes < w.bytes || (w.bytes > 0 && !ws)) return GGA_EWORKSPACE;
    w = carve(ws, n, e);
    hipStream_t s = as_stream(stream);

    if (e == 0 || n == 0) {
        fill_i32(row_ptr, (int64_t)n + 1, 0, s);
        if (e == 0) return launch_status();
    }

    const int64_t nblocks = (e + kRsTile - 1) / kRsTile;
    const Passes ps = passes_for(n);
    const int bits_total = key_bits(n);
    const int last = ps.count - 1;
    // values end in eid and others in col after the last pass: alternate so that they do
    int32_t* vbuf[2];
    int32_t* obuf[2];
    vbuf[last & 1] = eid;
    vbuf[(last & 1) ^ 1] = w.vals_tmp;
    obuf[last & 1] = col;
    obuf[(last & 1) ^ 1] = w.oth_tmp;
    for (int p = 0; p < ps.count; p++) {
        const int shift = ps.width * p;
        const int bits = (bits_total - shift) < ps.width ? (bits_total - shift) : ps.width;
        const int32_t* kin = p == 0 ? key : w.keys_tmp[(p - 1) & 1];
        const int32_t* vin = p == 0 ? nullptr : vbuf[(p - 1) & 1];
        const int32_t* oin = p == 0 ? other : obuf[(p - 1) & 1];
        int32_t* kout = w.keys_tmp[p & 1];
        radix_upsweep<<<(unsigned)nblocks, kRsThreads, 0, s>>>(kin, e, shift, bits, w.hist, nblocks);
        digit_rows_scan<<<1u << bits, kDsThreads, 0, s>>>(w.hist, nblocks, w.totals);
        // the last pass also writes row_ptr (n > 0; with no rows there is nothing to write)
        const bool rows = p == last && n > 0;
        RadixArgs a{kin, vin, oin, kout, vbuf[p & 1], obuf[p & 1], w.hist, w.totals, e, nblocks, shift, bits,
                    rows ? row_ptr : nullptr, w.run_key, w.run_pos, w.run_lkey, n};
        if (p == 0)
            radix_downsweep<true><<<(unsigned)nblocks, kRsThreads, 0, s>>>(a);
        else
            radix_downsweep<false><<<(unsigned)nblocks, kRsThreads, 0, s>>>(a);
        if (rows) {
            const int64_t runs = ((int64_t)1 << bits) * nblocks;
            row_ptr_gaps<<<grid_for((runs + kGapRuns - 1) / kGapRuns), 256, 0, s>>>(w.run_key, w.run_pos, w.run_lkey, w.hist, w.totals, bits,
                                                        nblocks, n, row_ptr);
        }
    }
    return launch_status();
}

extern "C" int gga_batch_edges(int32_t batch, const int32_t* node_ptr, const int32_t* edge_ptr, int64_t e,
                               const int32_t* src_local, const int32_t* dst_local, int32_t* src, int32_t* dst,
                               int32_t* d_bad, void* stream) {
    if (batch < 1 || e < 0) return GGA_EINVAL;
    if (e >= (int64_t)INT32_MAX) return GGA_ERANGE;
    if (!node_ptr || !edge_ptr || !d_bad || (e > 0 && (!src_local || !dst_local || !src || !dst))) return GGA_EINVAL;
    hipStream_t s = as_stream(stream);
    fill_i32(d_bad, 1, 0, s);
    if (e > 0) batch_edges_kernel<<<grid_for(e), 256, 0, s>>>(batch, node_ptr, edge_ptr, e, src_local, dst_local, src,
                                                              dst, d_bad);
    return launch_status();
}

extern "C" int gga_relation_sources(int32_t n, int32_t relations, int64_t e, const int32_t* src, const int32_t* dst,
                                    int32_t n_seg, const int32_t* seg, int32_t* src_rel, int32_t* d_bad,
                                    void* stream) {
    if (n < 0 || relations < 1 || e < 0 || n_seg < 0 || !d_bad) return GGA_EINVAL;
    if (e >= (int64_t)INT32_MAX || (int64_t)n * relations >= (int64_t)INT32_MAX) return GGA_ERANGE;
    if (e > 0 && (!src || !dst || !src_rel)) return GGA_EINVAL;
    if (n_seg > 0 && !seg) return GGA_EINVAL;
    int64_t pos = 0;
    for (int32_t k = 0; k < n_seg; k++) {
        const int32_t r = seg[3 * k], start = seg[3 * k + 1], end = seg[3 * k + 2];
        if (r < 0 || r >= relations || start != pos || end < start || end > e) return GGA_EINVAL;
        pos = end;
    }
    if (pos != e) return GGA_EINVAL;
    hipStream_t s = as_stream(stream);
    fill_i32(d_bad, 1, 0, s);
    for (int32_t k0 = 0; k0 < n_seg; k0 += kRelSegs) {
        RelSegs sg{};
        sg.count = n_seg - k0 < kRelSegs ? n_seg - k0 : kRelSegs;
        for (int k = 0; k < sg.count; k++) {
            sg.rel[k] = seg[3 * (k0 + k)];
            sg.start[k] = seg[3 * (k0 + k) + 1];
        }
        const int64_t lo = sg.start[0], hi = seg[3 * (k0 + sg.count - 1) + 2];
        if (hi > lo)
            relation_sources_kernel<<<grid_for(hi - lo), 256, 0, s>>>(n, relations, lo, hi, sg, src, dst, src_rel,
                                                                      d_bad);
    }
    return launch_status();
}
