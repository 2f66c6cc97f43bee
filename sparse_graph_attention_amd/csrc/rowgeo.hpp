// Lane geometry of a node row inside a wavefront, shared by the row kernels.
//
// A row of W = H*C elements is covered by LPR lanes holding EPL consecutive elements
// each; a head spans HDP lanes (C/EPL rounded up to a power of two; surplus lanes hold
// nothing); when H*HDP > 64 each lane holds NS slots, slot s covering row lanes
// s*64 .. s*64+63.  The 64/LPR groups of lanes in a wavefront work on different edges
// of the same row.
#pragma once

#include "common.hpp"

namespace gga {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Internal score mode: the additive logit plus a per-edge term read in CSR order.
constexpr int kScoreAddEdge = 3;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int EPL>
__device__ __forceinline__ void store_f32(float* dst, const float* f) {
    if constexpr (EPL == 8) {
        reinterpret_cast<float4*>(dst)[0] = make_float4(f[0], f[1], f[2], f[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(f[4], f[5], f[6], f[7]);
    } else if constexpr (EPL == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
    } else {
#pragma unroll
        for (int i = 0; i < EPL; i++) dst[i] = f[i];
    }
}

template <int EPL>
__device__ __forceinline__ void load_f32(const float* src, float* f) {
    if constexpr (EPL == 8) {
        const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else if constexpr (EPL == 4) {
        const float4 a = *reinterpret_cast<const float4*>(src);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; i++) f[i] = src[i];
    }
}

// load_f32 for a row the kernel reads once (non-temporal hint).
template <int EPL>
__device__ __forceinline__ void load_f32_once(const float* src, float* f) {
    if constexpr (EPL == 8 || EPL == 4) {
#pragma unroll
        for (int h = 0; h < EPL / 4; h++) {
            const float4 a = load_once(reinterpret_cast<const float4*>(src) + h);
            f[4 * h] = a.x; f[4 * h + 1] = a.y; f[4 * h + 2] = a.z; f[4 * h + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPL; i++) f[i] = load_once(src + i);
    }
}

template <int EPL, int HDP, int NS>
struct RowGeo {
    int lane, g, G, lpr;
    int off[NS], head[NS];
    bool ok[NS], lead[NS];
    bool exact;  // one slot, and the lpr lanes of a group cover the row exactly


    __device__ __forceinline__ void init(int lpr_log2, int H, int C) {
        lane = threadIdx.x & 63;
        lpr = 1 << lpr_log2;
        G = 64 >> lpr_log2;
        g = lane >> lpr_log2;
        const int li = lane & (lpr - 1);
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const int j = s * 64 + li;
            head[s] = j / HDP;
            const int sub = j % HDP;
            ok[s] = head[s] < H && sub * EPL < C;
            off[s] = head[s] * C + sub * EPL;
            lead[s] = sub == 0;
        }
        exact = NS == 1 && lpr == H * HDP && HDP * EPL == C;
    }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Stores a node's output row held by the lanes of group 0 (lane l holds elements
// [l*EPL, (l+1)*EPL) of a row of lpr*EPL floats) with non-temporal stores that each cover
// consecutive 16-byte chunks of the row.  With 8 floats per lane the chunks are first
// exchanged across lanes so that one store instruction writes a contiguous 1 KiB instead
// of half of every cache line twice.  All 64 lanes must call it (it shuffles).
template <int EPL>
__device__ __forceinline__ void store_row_nt(float* row, const float* vals, int lpr, int lane, int g) {
    if constexpr (EPL == 8) {
        const int nchunks = lpr * 2;
        for (int base = 0; base < nchunks; base += 64) {
            const int c = base + lane;
            const int srcl = (c >> 1) & 63;
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = __shfl(vals[i], srcl, 64);
                b[i] = __shfl(vals[4 + i], srcl, 64);
            }
            if (c < nchunks) {
                const f32x4 val = (c & 1) ? f32x4{b[0], b[1], b[2], b[3]} : f32x4{a[0], a[1], a[2], a[3]};
                __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(row) + c);
            }
        }
    } else if constexpr (EPL == 4) {
        if (g == 0)
            __builtin_nontemporal_store(f32x4{vals[0], vals[1], vals[2], vals[3]},
                                        reinterpret_cast<f32x4*>(row) + lane);
    } else {
        if (g == 0)
#pragma unroll
            for (int i = 0; i < EPL; i++) __builtin_nontemporal_store(vals[i], row + lane * EPL + i);
    }
}

// Stores, for every group of lpr lanes, the output row that group holds (lane l of the
// group holds elements [l*EPL, (l+1)*EPL) of a row of lpr*EPL floats at `row`, which
// differs by group) with non-temporal stores covering consecutive 16-byte chunks; with 8
// floats per lane the chunks are exchanged within the group first.  All 64 lanes must
// call it; a group with `valid` false stores nothing.
template <int EPL>
__device__ __forceinline__ void store_group_row_nt(float* row, const float* vals, int lpr, int lane, bool valid) {
    const int gl = lane & (lpr - 1), g0 = lane - gl;
    if constexpr (EPL == 8) {
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const int c = k * lpr + gl;
            const int srcl = g0 + (c >> 1);
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = __shfl(vals[i], srcl, 64);
                b[i] = __shfl(vals[4 + i], srcl, 64);
            }
            const f32x4 val = (c & 1) ? f32x4{b[0], b[1], b[2], b[3]} : f32x4{a[0], a[1], a[2], a[3]};
            if (valid) __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(row) + c);
        }
    } else if constexpr (EPL == 4) {
        if (valid)
            __builtin_nontemporal_store(f32x4{vals[0], vals[1], vals[2], vals[3]}, reinterpret_cast<f32x4*>(row) + gl);
    } else {
        if (valid)
#pragma unroll
            for (int i = 0; i < EPL; i++) __builtin_nontemporal_store(vals[i], row + gl * EPL + i);
    }
}

// Sum of a value over the G edge groups of a wavefront (butterfly from LPR up to 32).
__device__ __forceinline__ float sum_groups(float x, int lpr) {
    for (int o = lpr; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace gga
