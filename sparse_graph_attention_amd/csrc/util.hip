// Fill and exclusive-scan primitives used by the CSR build and the degree plan.
#include "common.hpp"

namespace gga {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;  // 4096

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t value) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float value) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

__device__ __forceinline__ int pad(int i) { return i + (i >> 4); }

// Inclusive scan across a wavefront.
__device__ __forceinline__ int wave_inclusive(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Exclusive scan of one value per thread over the 256-thread block; returns the block total.
__device__ int block_exclusive(int x, int* excl, int* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = wave_inclusive(x);
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; w++) {
        int t = wave_tot[w];
        before += (w < wave) ? t : 0;
        total += t;
    }
    *excl = before + inc - x;
    return total;
}

// Column blockIdx.y of the scan: each launch scans all columns of a ScanCols together.
__global__ void scan_reduce(ScanCols sc, int64_t n, int32_t* bsum, int64_t nb) {
    __shared__ int wave_tot[kScanThreads / 64];
    const int32_t* in = sc.col[blockIdx.y];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; k++) {
        int64_t i = base + k * kScanThreads + threadIdx.x;
        s += (i < n) ? in[i] : 0;
    }
    int excl;
    int tot = block_exclusive(s, &excl, wave_tot);
    if (threadIdx.x == 0) bsum[blockIdx.y * nb + blockIdx.x] = tot;
}

// One block per column: exclusive scan of that column's block sums in place, its total
// to total[column] when given.
__global__ void scan_block_sums(ScanCols sc, int32_t* bsum_all, int64_t nb) {
    __shared__ int wave_tot[kScanThreads / 64];
    int32_t* bsum = bsum_all + blockIdx.x * nb;
    int carry = 0;
    for (int64_t base = 0; base < nb; base += kScanThreads) {
        int64_t i = base + threadIdx.x;
        int x = (i < nb) ? bsum[i] : 0;
        int excl;
        int tot = block_exclusive(x, &excl, wave_tot);
        if (i < nb) bsum[i] = carry + excl;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0 && sc.total[blockIdx.x]) *sc.total[blockIdx.x] = carry;
}

__global__ void scan_down(ScanCols sc, int64_t n, const int32_t* bsum, int64_t nb) {
    __shared__ int lds[kScanTile + kScanTile / 16];
    __shared__ int wave_tot[kScanThreads / 64];
    int32_t* col = sc.col[blockIdx.y];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll
    for (int k = 0; k < kScanItems; k++) {
        int idx = k * kScanThreads + threadIdx.x;
        int64_t i = base + idx;
        lds[pad(idx)] = (i < n) ? col[i] : 0;
    }
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; j++) s += lds[pad(threadIdx.x * kScanItems + j)];
    int excl;
    block_exclusive(s, &excl, wave_tot);
    int run = bsum[blockIdx.y * nb + blockIdx.x] + excl;
#pragma unroll
    for (int j = 0; j < kScanItems; j++) {
        int p = pad(threadIdx.x * kScanItems + j);
        int v = lds[p];
        lds[p] = run;
        run += v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScanItems; k++) {
        int idx = k * kScanThreads + threadIdx.x;
        int64_t i = base + idx;
        if (i < n) col[i] = lds[pad(idx)];
    }
}

int grid_for(int64_t n, int threads) {
    int64_t b = (n + threads - 1) / threads;
    if (b < 1) b = 1;
    if (b > 65536) b = 65536;
    return (int)b;
}

}  // namespace

void fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t s) {
    if (n <= 0) return;
    fill_i32_kernel<<<grid_for(n, 256), 256, 0, s>>>(p, n, value);
}

void fill_f32(float* p, int64_t n, float value, hipStream_t s) {
    if (n <= 0) return;
    fill_f32_kernel<<<grid_for(n, 256), 256, 0, s>>>(p, n, value);
}

size_t scan_workspace_elems(int64_t n) { return (size_t)kScanMaxCols * ((n + kScanTile - 1) / kScanTile) + 1; }

void exclusive_scan_cols(const ScanCols& sc, int64_t n, int32_t* scratch, hipStream_t s) {
    if (sc.ncols <= 0) return;
    if (n <= 0) {
        for (int c = 0; c < sc.ncols; c++)
            if (sc.total[c]) fill_i32(sc.total[c], 1, 0, s);
        return;
    }
    int64_t nb = (n + kScanTile - 1) / kScanTile;
    const dim3 grid((unsigned)nb, (unsigned)sc.ncols);
    scan_reduce<<<grid, kScanThreads, 0, s>>>(sc, n, scratch, nb);
    scan_block_sums<<<(unsigned)sc.ncols, kScanThreads, 0, s>>>(sc, scratch, nb);
    scan_down<<<grid, kScanThreads, 0, s>>>(sc, n, scratch, nb);
}

}  // namespace gga
