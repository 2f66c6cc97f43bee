// Shared device helpers of libgga (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gga.h"

namespace gga {

constexpr int kWave = 64;

// MI355X hands the workgroups of a launch to its 8 XCDs round-robin by linear id, and each
// XCD has its own L2.  xcd_order maps a linear id so that each XCD receives one contiguous
// range of the logical order: workgroups that share operands then share an L2.  A
// bijection on [0, total) for any total.
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_order(uint32_t lin, uint32_t total) {
    const uint32_t xcd = lin % kXcds, j = lin / kXcds;
    const uint32_t q = total / kXcds, r = total % kXcds;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + j;
}

// Orders a wavefront's LDS writes before later LDS reads of the same locations by other
// lanes of that wavefront.  The hardware completes one wavefront's LDS operations in
// order, so nothing waits; the wavefront-scope fences keep the compiler from moving
// memory operations across the point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A row piece of 16, 8 or 4 bytes loaded with the non-temporal hint: for rows a kernel reads
// once (the row it owns), so that they displace fewer of the rows it gathers again.
template <typename R>
__device__ __forceinline__ R load_once(const R* p) {
    if constexpr (sizeof(R) == 16) {
        typedef uint32_t u4v __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p)));
    } else if constexpr (sizeof(R) == 8) {
        typedef uint32_t u2v __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const u2v*>(p)));
    } else if constexpr (sizeof(R) == 4) {
        return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)));
    } else {
        return *p;
    }
}

// ---------------------------------------------------------------- host helpers

inline int launch_status() { return hipGetLastError() == hipSuccess ? GGA_OK : GGA_EHIP; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Carves consecutive 256-byte aligned sub-buffers out of a workspace.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t count) {
        off = align_up(off, 256);
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += count * sizeof(T);
        return p;
    }
    size_t bytes() const { return align_up(off, 256); }
};

// ---------------------------------------------------------------- element types

struct bf16x8 {
    uint4 raw;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Vector of EPL elements of storage type T loaded from 16/8/4/2 bytes and widened to fp32.
template <typename T, int EPL>
struct Vec;

template <>
struct Vec<float, 4> {
    using raw_t = float4;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) {
        f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
    }
};
template <>
struct Vec<float, 2> {
    using raw_t = float2;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) { f[0] = r.x; f[1] = r.y; }
};
template <>
struct Vec<float, 1> {
    using raw_t = float;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) { f[0] = r; }
};
template <>
struct Vec<uint16_t, 8> {
    using raw_t = uint4;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
};
template <>
struct Vec<uint16_t, 4> {
    using raw_t = uint2;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    }
};
template <>
struct Vec<uint16_t, 2> {
    using raw_t = uint32_t;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) { f[0] = bf16_lo(r); f[1] = bf16_hi(r); }
};
template <>
struct Vec<uint16_t, 1> {
    using raw_t = uint16_t;
    static __device__ __forceinline__ void widen(const raw_t& r, float* f) { f[0] = __uint_as_float(uint32_t(r) << 16); }
};

// ---------------------------------------------------------------- cross-lane

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// DPP controls on gfx9: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float swz_xor16(float x) {
    // ds_swizzle in bit mode: and_mask 0x1f, or 0, xor 0x10 (within 32-lane halves)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (0x10 << 10) | 0x1f));
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of the group
// receives the group's sum.  The combination order is fixed, so results are reproducible.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G > 1) x += dpp_f<kDppXor1>(x);
    if constexpr (G > 2) x += dpp_f<kDppXor2>(x);
    if constexpr (G > 4) x += dpp_f<kDppHalfMirror>(x);
    if constexpr (G > 8) x += dpp_f<kDppMirror>(x);
    if constexpr (G > 16) x += swz_xor16(x);
    if constexpr (G > 32) x += __shfl_xor(x, 32, 64);
    return x;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- kernels shared by files

// Fill n int32 with a value (used instead of hipMemsetAsync so that every call is a kernel).
void fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t s);
void fill_f32(float* p, int64_t n, float value, hipStream_t s);

// Exclusive prefix sums, in place, of up to kScanMaxCols int32 columns of n entries each,
// all in the same three launches; column c's total goes to *total[c] (device) when total[c]
// is not null.  Needs scan_workspace_elems(n) int32 of scratch.
constexpr int kScanMaxCols = 5;

struct ScanCols {
    int32_t* col[kScanMaxCols];
    int32_t* total[kScanMaxCols];
    int ncols;
};

size_t scan_workspace_elems(int64_t n);
void exclusive_scan_cols(const ScanCols& sc, int64_t n, int32_t* scratch, hipStream_t s);

}  // namespace gga
