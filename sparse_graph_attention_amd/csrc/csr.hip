// COO -> CSR by key: a stable least-significant-digit radix sort of (key, COO index,
// other endpoint).
//
// A build takes ceil(bits / 8) passes over the key bits (three for n <= 2^24), each sorting
// by one digit of at most 8 bits.  A pass is stable by construction: each wavefront of a
// tile ranks its own contiguous run of items in their original order (64 at a time, the
// lanes with equal digits found by ballots, a per-digit running count in LDS carrying over
// from one 64-item round to the next), the wavefronts' runs are placed in wavefront order
// (per-digit counts of each wavefront, scanned in LDS), and tiles are ordered by a
// digit-major exclusive scan of per-tile histograms.  The result therefore equals a stable
// sort, independent of scheduling: within a row the COO indices ascend, bit-exact across
// runs and devices.  The other endpoint travels with each item, so the last pass writes
// col directly.  Each tile is staged in LDS in digit order before it is written, so the
// scatter writes contiguous runs.  row_ptr comes from the segment boundaries of the sorted
// keys; no atomics decide any position.
#include "common.hpp"

namespace gga {

namespace {

constexpr int kMaxDigitBits = 8;
constexpr int kMaxBins = 1 << kMaxDigitBits;
constexpr int kRsWaves = 4;
constexpr int kRsThreads = 64 * kRsWaves;
constexpr int kRsRounds = 16;                    // 64-item rounds per wavefront
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

// Lanes of the wavefront whose item is valid and has digit d (as this lane's).
__device__ __forceinline__ uint64_t same_digit_lanes(uint32_t d, bool valid, int bits) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; b++) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    return peers;
}

// Per-tile digit counts: hist[d * nblocks + tile].
__global__ __launch_bounds__(kRsThreads) void radix_upsweep(const int32_t* __restrict__ keys, int64_t e, int shift,
                                                            int bits, int32_t* __restrict__ hist, int64_t nblocks) {
    __shared__ int cnt[kMaxBins];
    const int bins = 1 << bits;
    const uint32_t mask = (uint32_t)bins - 1u;
    for (int d = threadIdx.x; d < bins; d += kRsThreads) cnt[d] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRsTile;
    int32_t k[kRsRounds];
#pragma unroll
    for (int r = 0; r < kRsRounds; r++) {
        const int64_t i = base + r * kRsThreads + threadIdx.x;
        k[r] = i < e ? keys[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kRsRounds; r++) {
        const int64_t i = base + r * kRsThreads + threadIdx.x;
        if (i < e) atomicAdd(&cnt[digit_of(k[r], shift, mask)], 1);
    }
    __syncthreads();
    for (int d = threadIdx.x; d < bins; d += kRsThreads) hist[(int64_t)d * nblocks + blockIdx.x] = cnt[d];
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
    const int32_t* offsets;  // digit-major exclusive scan of the per-tile digit counts
    int64_t e, nblocks;
    int shift, bits;
};

struct RadixSmem {
    // a wavefront's 16-bit per-digit counts, then its next tile position per digit; digit d
    // sits in half d & 1 of word d / 2 (positions stay below 2^16, so halves never carry)
    uint32_t wpos[kRsWaves][kMaxBins / 2];
    uint16_t tdo[kMaxBins];   // tile-local start of each digit
    int32_t gbase[kMaxBins];  // global start of each digit's run of this tile
    int32_t wtot[kRsWaves];
    int32_t skey[kRsTile];
    int32_t sval[kRsTile];
    int32_t soth[kRsTile];
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
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int i = tid; i < kRsWaves * (kMaxBins / 2); i += kRsThreads) {
        const int w = i / (kMaxBins / 2), x = i % (kMaxBins / 2);
        if (x < words) sm.wpos[w][x] = 0;
    }
    __syncthreads();  // (also: the previous tile's scatter has read tdo, gbase and the staging)

    // each wavefront counts its digits (additions commute: no ordering needed)
#pragma unroll
    for (int r = 0; r < kRsRounds; r++) {
        const bool valid = wbase + r * 64 + lane < tile_n;
        const uint32_t d = digit_of(it.key[r], shift, mask);
        if (valid) atomicAdd(&sm.wpos[wave][d >> 1], 1u << (16 * (d & 1)));
    }
    __syncthreads();

    // tile-local digit starts (scan over digits), each wavefront's start per digit (in
    // wavefront order), and the global start of each digit's run of this tile.  A thread
    // owns kDigitsPerThread consecutive digits, i.e. whole words of wpos.
    {
        int c[kDigitsPerThread];
        int tot = 0;
#pragma unroll
        for (int j = 0; j < kDigitsPerThread; j++) {
            const int d = tid * kDigitsPerThread + j;
            c[j] = 0;
            if (d < bins)
                for (int w = 0; w < kRsWaves; w++) c[j] += (sm.wpos[w][d >> 1] >> (16 * (d & 1))) & 0xffffu;
            tot += c[j];
        }
        int x = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) sm.wtot[wave] = x;
        __syncthreads();
        int run = x - tot;
        for (int w = 0; w < wave; w++) run += sm.wtot[w];
#pragma unroll
        for (int m = 0; m < kDigitsPerThread / 2; m++) {
            const int d0 = tid * kDigitsPerThread + 2 * m;
            if (d0 < bins) {
                uint32_t s0 = (uint32_t)run, s1 = (uint32_t)(run + c[2 * m]);
                sm.tdo[d0] = (uint16_t)s0;
                sm.gbase[d0] = a.offsets[(int64_t)d0 * a.nblocks + tile];
                if (d0 + 1 < bins) {
                    sm.tdo[d0 + 1] = (uint16_t)s1;
                    sm.gbase[d0 + 1] = a.offsets[(int64_t)(d0 + 1) * a.nblocks + tile];
                }
                for (int w = 0; w < kRsWaves; w++) {
                    const uint32_t cw = sm.wpos[w][d0 >> 1];
                    sm.wpos[w][d0 >> 1] = s0 | (s1 << 16);
                    s0 += cw & 0xffffu;
                    s1 += cw >> 16;
                }
            }
            run += c[2 * m] + c[2 * m + 1];
        }
    }
    __syncthreads();

    // each wavefront places its items in order.  Per round the lowest lane of each group of
    // equal digits takes the group's places with one atomic add that returns the digit's
    // next position; a wavefront's LDS operations complete in issue order, so the rounds'
    // adds follow one another and every group lands after the earlier rounds' items of its
    // digit.  The group's members take the returned start from their lowest lane.
    // (in two halves of kRsRounds / 2 rounds, to bound the registers holding the returns)
#pragma unroll
    for (int h = 0; h < 2; h++) {
        constexpr int kHalf = kRsRounds / 2;
        uint32_t got[kHalf], rl[kHalf];  // rl: rank in the group | lowest lane << 8
#pragma unroll
        for (int q = 0; q < kHalf; q++) {
            const int r = h * kHalf + q;
            const bool valid = wbase + r * 64 + lane < tile_n;
            const uint32_t d = digit_of(it.key[r], shift, mask);
            const uint64_t peers = same_digit_lanes(d, valid, bits);
            const uint32_t rank = (uint32_t)__popcll(peers & below);
            got[q] = 0;
            rl[q] = rank | ((uint32_t)(valid ? __ffsll((unsigned long long)peers) - 1 : lane) << 8);
            if (valid && rank == 0)
                got[q] = atomicAdd(&sm.wpos[wave][d >> 1], (uint32_t)__popcll(peers) << (16 * (d & 1)));
        }
#pragma unroll
        for (int q = 0; q < kHalf; q++) {
            const int r = h * kHalf + q;
            const bool valid = wbase + r * 64 + lane < tile_n;
            const uint32_t d = digit_of(it.key[r], shift, mask);
            const uint32_t w0 = (uint32_t)__shfl((int)got[q], (int)(rl[q] >> 8), 64);
            if (valid) {
                const int pos = (int)((w0 >> (16 * (d & 1))) & 0xffffu) + (int)(rl[q] & 0xffu);
                sm.skey[pos] = it.key[r];
                sm.sval[pos] = it.val[r];
                sm.soth[pos] = it.oth[r];
            }
        }
    }
    __syncthreads();

    // the tile now sits in LDS in (digit, original order); write each digit's run contiguously
    for (int li = tid; li < tile_n; li += kRsThreads) {
        const int32_t k = sm.skey[li];
        const uint32_t d = digit_of(k, shift, mask);
        const int64_t pos = (int64_t)sm.gbase[d] + (li - (int)sm.tdo[d]);
        if (a.keys_out) a.keys_out[pos] = k;
        a.vals_out[pos] = sm.sval[li];
        a.oth_out[pos] = sm.soth[li];
    }
    (void)base;
}

// One pass: one workgroup per tile.
template <bool FIRST>
__global__ __launch_bounds__(kRsThreads) void radix_downsweep(RadixArgs a) {
    __shared__ RadixSmem sm;
    TileItems x;
    load_tile<FIRST>(a, blockIdx.x, x);
    sort_tile(a, blockIdx.x, x, sm);
}

// row_ptr from the sorted keys: row_ptr[v] = first position whose key is >= v.  Position p
// writes the rows v in (key[p-1], key[p]] (clamped to [0, n]); every write is in bounds even
// when keys are out of range.  A thread takes kRowPtrItems consecutive positions.
constexpr int kRowPtrItems = 4;

__global__ void row_ptr_from_sorted(const int32_t* __restrict__ skeys, int64_t e, int32_t n,
                                    int32_t* __restrict__ row_ptr) {
    const int64_t groups = (e + 1 + kRowPtrItems - 1) / kRowPtrItems;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < groups;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p0 = t * kRowPtrItems;
        int64_t kp = p0 > 0 ? (int64_t)skeys[p0 - 1] : -1;
        int64_t kc[kRowPtrItems];
#pragma unroll
        for (int j = 0; j < kRowPtrItems; j++) kc[j] = p0 + j < e ? (int64_t)skeys[p0 + j] : (int64_t)n;
#pragma unroll
        for (int j = 0; j < kRowPtrItems; j++) {
            const int64_t p = p0 + j;
            if (p > e) break;
            const int64_t lo = kp + 1 < 0 ? 0 : kp + 1;
            const int64_t hi = kc[j] < n ? kc[j] : n;
            for (int64_t v = lo; v <= hi; v++) row_ptr[v] = (int32_t)p;
            kp = kc[j];
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
    int32_t* scan;
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
    w.scan = c.take<int32_t>(scan_workspace_elems(hist_n > n ? hist_n : n));
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
        exclusive_scan_i32(w.hist, w.hist, ((int64_t)1 << bits) * nblocks, nullptr, w.scan, s);
        RadixArgs a{kin, vin, oin, kout, vbuf[p & 1], obuf[p & 1], w.hist, e, nblocks, shift, bits};
        if (p == 0)
            radix_downsweep<true><<<(unsigned)nblocks, kRsThreads, 0, s>>>(a);
        else
            radix_downsweep<false><<<(unsigned)nblocks, kRsThreads, 0, s>>>(a);
    }
    if (n > 0)
        row_ptr_from_sorted<<<grid_for((e + kRowPtrItems) / kRowPtrItems), 256, 0, s>>>(w.keys_tmp[last & 1], e, n,
                                                                                      row_ptr);
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
