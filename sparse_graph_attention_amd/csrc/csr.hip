// COO -> CSR by key: a stable least-significant-digit radix sort of (key, COO index).
//
// Each pass sorts by 8 bits of the key.  A pass is stable by construction: a tile's
// items are ranked in their original order (wave ballots give the rank among equal
// digits inside a wave, per-wave counts in LDS order the waves, a running per-digit
// count orders the rounds) and tiles are ordered by a digit-major exclusive scan of
// per-tile histograms.  The result therefore equals a stable sort, independent of
// scheduling: within a row the COO indices ascend, bit-exact across runs and devices.
// Each tile's items are staged in LDS in digit order before they are written, so the
// scatter writes contiguous runs.  row_ptr comes from the segment boundaries of the
// sorted keys; no atomics take part in the build.
#include "common.hpp"

namespace gga {

namespace {

constexpr int kRsThreads = 256;
constexpr int kRsItems = 16;
constexpr int kRsTile = kRsThreads * kRsItems;  // 4096 edges per tile
constexpr int kRsBins = 256;
constexpr int kRsWaves = kRsThreads / 64;

__global__ void count_bad(const int32_t* __restrict__ a, const int32_t* __restrict__ b, int64_t e, int32_t n,
                          int32_t* __restrict__ bad) {
    int local = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < e; i += (int64_t)gridDim.x * blockDim.x)
        local += ((uint32_t)a[i] >= (uint32_t)n) + ((uint32_t)b[i] >= (uint32_t)n);
    if (local) atomicAdd(bad, local);
}

__global__ void radix_upsweep(const int32_t* __restrict__ keys, int64_t e, int shift, uint32_t mask,
                              int32_t* __restrict__ hist, int64_t nblocks) {
    __shared__ int cnt[kRsBins];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRsTile;
#pragma unroll 4
    for (int k = 0; k < kRsItems; k++) {
        int64_t i = base + k * kRsThreads + threadIdx.x;
        if (i < e) atomicAdd(&cnt[((uint32_t)keys[i] >> shift) & mask], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * nblocks + blockIdx.x] = cnt[threadIdx.x];
}

// vals_in == nullptr means the identity (COO index).  `offsets` is the digit-major exclusive
// scan of the per-tile digit counts (offsets[d * nblocks + b]); `total` = e.
__global__ __launch_bounds__(kRsThreads) void radix_downsweep(const int32_t* __restrict__ keys_in,
                                                              const int32_t* __restrict__ vals_in,
                                                              int32_t* __restrict__ keys_out,
                                                              int32_t* __restrict__ vals_out, int64_t e, int shift,
                                                              int bits, const int32_t* __restrict__ offsets,
                                                              int64_t nblocks) {
    __shared__ int run[kRsBins];    // items of each digit placed so far in this tile
    __shared__ int tdo[kRsBins];    // tile-local start of each digit
    __shared__ int gbase[kRsBins];  // global start of each digit's run of this tile
    __shared__ int wc[kRsWaves][kRsBins];
    __shared__ int wtot[kRsWaves];
    __shared__ int32_t skey[kRsTile];
    __shared__ int32_t sval[kRsTile];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t base = (int64_t)blockIdx.x * kRsTile;
    const int tile_n = (int)((e - base) < kRsTile ? (e - base) : kRsTile);
    // this tile's count of digit tid, from the scan's neighbour (the scan is over a flat array)
    const int64_t oi = (int64_t)tid * nblocks + blockIdx.x;
    const int g0 = offsets[oi];
    const int g1 = (oi + 1 < (int64_t)kRsBins * nblocks) ? offsets[oi + 1] : (int)e;
    const int cnt = g1 - g0;
    gbase[tid] = g0;
    run[tid] = 0;
    {  // exclusive scan of the tile counts over the digits
        int x = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wtot[wave] = x;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; w++) before += wtot[w];
        tdo[tid] = before + x - cnt;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r = 0; r < kRsItems; r++) {
        const int li = r * kRsThreads + tid;
        const bool valid = li < tile_n;
        const int32_t key = valid ? keys_in[base + li] : 0;
        const int32_t val = valid ? (vals_in ? vals_in[base + li] : (int32_t)(base + li)) : 0;
        const uint32_t d = ((uint32_t)key >> shift) & mask;
#pragma unroll
        for (int w = 0; w < kRsWaves; w++) wc[w][tid] = 0;
        __syncthreads();
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; b++) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        const int rank = __popcll(peers & lt);
        if (valid && rank == 0) wc[wave][d] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int pos = tdo[d] + run[d] + rank;
            for (int w = 0; w < wave; w++) pos += wc[w][d];
            skey[pos] = key;
            sval[pos] = val;
        }
        __syncthreads();
        int add = 0;
#pragma unroll
        for (int w = 0; w < kRsWaves; w++) add += wc[w][tid];
        run[tid] += add;
    }
    __syncthreads();
    // the tile now sits in LDS in (digit, original order); write each digit's run contiguously
    for (int li = tid; li < tile_n; li += kRsThreads) {
        const int32_t key = skey[li];
        const uint32_t d = ((uint32_t)key >> shift) & mask;
        const int pos = gbase[d] + (li - tdo[d]);
        if (keys_out) keys_out[pos] = key;
        vals_out[pos] = sval[li];
    }
}

// row_ptr from the sorted keys: row_ptr[v] = first position whose key is >= v.  Position p
// writes the rows v in (key[p-1], key[p]] (clamped to [0, n]); every write is in bounds even
// when keys are out of range.
__global__ void row_ptr_from_sorted(const int32_t* __restrict__ skeys, int64_t e, int32_t n,
                                    int32_t* __restrict__ row_ptr) {
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p <= e; p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t kp = p > 0 ? (int64_t)skeys[p - 1] : -1;
        const int64_t kc = p < e ? (int64_t)skeys[p] : (int64_t)n;
        const int64_t lo = kp + 1 < 0 ? 0 : kp + 1;
        const int64_t hi = kc < n ? kc : n;
        for (int64_t v = lo; v <= hi; v++) row_ptr[v] = (int32_t)p;
    }
}

__global__ void gather_col(const int32_t* __restrict__ other, const int32_t* __restrict__ eid, int64_t e,
                           int32_t* __restrict__ col) {
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < e; p += (int64_t)gridDim.x * blockDim.x)
        col[p] = other[eid[p]];
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

struct CsrWs {
    int32_t* hist;
    int32_t* scan;
    int32_t* keys_tmp;
    int32_t* vals_tmp;
    size_t bytes;
};

CsrWs carve(void* ws, int32_t n, int64_t e) {
    Carver c(ws);
    CsrWs w;
    int64_t nblocks = (e + kRsTile - 1) / kRsTile;
    int64_t hist_n = (int64_t)kRsBins * nblocks;
    w.hist = c.take<int32_t>((size_t)hist_n);
    size_t sc = scan_workspace_elems(hist_n > n ? hist_n : n);
    w.scan = c.take<int32_t>(sc);
    w.keys_tmp = c.take<int32_t>((size_t)e);
    w.vals_tmp = c.take<int32_t>((size_t)e);
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
    const int bits_total = key_bits(n);
    const int passes = bits_total == 0 ? 1 : (bits_total + 7) / 8;
    const int last = passes - 1;
    int32_t* kbuf[2] = {w.keys_tmp, col};  // col is free until the final gather
    int32_t* vbuf[2];
    vbuf[last & 1] = eid;
    vbuf[(last & 1) ^ 1] = w.vals_tmp;
    for (int p = 0; p < passes; p++) {
        const int shift = 8 * p;
        const int bits = bits_total == 0 ? 0 : ((bits_total - shift) < 8 ? (bits_total - shift) : 8);
        const uint32_t mask = (1u << bits) - 1u;
        const int32_t* kin = p == 0 ? key : kbuf[(p - 1) & 1];
        const int32_t* vin = p == 0 ? nullptr : vbuf[(p - 1) & 1];
        int32_t* kout = kbuf[p & 1];
        int32_t* vout = vbuf[p & 1];
        radix_upsweep<<<(unsigned)nblocks, kRsThreads, 0, s>>>(kin, e, shift, mask, w.hist, nblocks);
        exclusive_scan_i32(w.hist, w.hist, (int64_t)kRsBins * nblocks, nullptr, w.scan, s);
        radix_downsweep<<<(unsigned)nblocks, kRsThreads, 0, s>>>(kin, vin, kout, vout, e, shift, bits, w.hist,
                                                                  nblocks);
    }
    if (n > 0) row_ptr_from_sorted<<<grid_for(e + 1), 256, 0, s>>>(kbuf[last & 1], e, n, row_ptr);
    gather_col<<<grid_for(e), 256, 0, s>>>(other, eid, e, col);
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
