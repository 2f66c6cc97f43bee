// Global linear-attention branch ("Gated Local-Global Graph Attention", Key formulas G_i,
// S, z; Implementation notes item 2, phi = elu + 1), forward and backward, per head h of width r:
//   S[h] = sum_j phi(k_j) v_j^T,  z[h] = sum_j phi(k_j),
//   G[i] = phi(q_i)^T S[h] / (phi(q_i) . z[h] + eps).
// The sums over j run over a fixed split of the node axis (one partial per range) that a
// second kernel adds in range order.  For r a multiple of 16 (up to 64) both contractions
// run on the matrix cores (v_mfma_f32_16x16x4_f32); other widths take a scalar path.
#include "common.hpp"

namespace gga {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// N consecutive floats (N = 1..4) in one load; p must be 4*N-byte aligned (16 for N = 3).
template <int N>
__device__ __forceinline__ void load_n(const float* p, float* out) {
    if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        out[0] = t.x; out[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = p[i];
    }
}

template <int N>
__device__ __forceinline__ void store_n(float* p, const float* v) {
    if constexpr (N == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) p[i] = v[i];
    }
}

// Number of node ranges of the statistics (a function of n only, so the order of the
// sums is fixed): ranges of at least 256 nodes, at most 1024 ranges.
int row_ranges(int32_t n) {
    int64_t nb = ((int64_t)n + 255) / 256;
    if (nb < 1) nb = 1;
    if (nb > 1024) nb = 1024;
    return (int)nb;
}

// ---- statistics, matrix-core path.  grid nb; a workgroup owns one node range and has one
// wavefront per head (up to 16; more heads loop), so the wavefronts of a workgroup read the
// same rows together.  Each step takes 4 rows (lane / 16); four steps are loaded before any
// is multiplied.
template <int TR>
__global__ __launch_bounds__(1024) void stats_mfma(int32_t n, int32_t H, int32_t rows_per, const float* __restrict__ k,
                                                   const float* __restrict__ v, float* __restrict__ part) {
    constexpr int R = TR * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int64_t W = (int64_t)H * R;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per;
    const int64_t r1 = r0 + rows_per < n ? r0 + rows_per : n;
    for (int h = wave; h < H; h += nw) {
        v4f acc[TR][TR];
        float zacc[TR];
#pragma unroll
        for (int i = 0; i < TR; i++) {
            zacc[i] = 0.f;
#pragma unroll
            for (int j = 0; j < TR; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        // Feature order inside a head is permuted: MFMA tile u, position p <-> feature
        // TR*p + u, so lane p loads its TR features of a row as one vector.
        for (int64_t base = r0; base < r1; base += 16) {
            float a[4][TR], b[4][TR];
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const int64_t row = base + st * 4 + (lane >> 4);
                if (row < r1) {
                    const int64_t o = row * W + h * R + TR * (lane & 15);
                    load_n<TR>(k + o, a[st]);
                    load_n<TR>(v + o, b[st]);
#pragma unroll
                    for (int t = 0; t < TR; t++) a[st][t] = phi(a[st][t]);
                } else {
#pragma unroll
                    for (int t = 0; t < TR; t++) a[st][t] = b[st][t] = 0.f;
                }
            }
#pragma unroll
            for (int st = 0; st < 4; st++) {
#pragma unroll
                for (int t = 0; t < TR; t++) zacc[t] += a[st][t];
#pragma unroll
                for (int i = 0; i < TR; i++)
#pragma unroll
                    for (int j = 0; j < TR; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st][i], b[st][j], acc[i][j], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < TR; t++) {
            zacc[t] += __shfl_xor(zacc[t], 16, 64);
            zacc[t] += __shfl_xor(zacc[t], 32, 64);
        }
        float* out = part + ((int64_t)blockIdx.x * H + h) * (R * R + R);
        // acc[i][j][q] of lane l is S[TR*pi + i][TR*pj + j] with pi = (l/16)*4 + q, pj = l%16
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int pi = (lane >> 4) * 4 + q, pj = lane & 15;
#pragma unroll
            for (int i = 0; i < TR; i++) {
                float row[TR];
#pragma unroll
                for (int j = 0; j < TR; j++) row[j] = acc[i][j][q];
                store_n<TR>(out + (TR * pi + i) * R + TR * pj, row);
            }
        }
        if (lane < 16) store_n<TR>(out + R * R + TR * lane, zacc);
    }
}

// ---- statistics, scalar path (any r).  grid (nb, H); threads over the r*r + r outputs.
__global__ __launch_bounds__(256) void stats_scalar(int32_t n, int32_t H, int32_t R, int32_t rows_per,
                                                    const float* __restrict__ k, const float* __restrict__ v,
                                                    float* __restrict__ part) {
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per;
    const int64_t r1 = r0 + rows_per < n ? r0 + rows_per : n;
    float* out = part + ((int64_t)blockIdx.x * H + h) * (R * R + R);
    for (int e = threadIdx.x; e < R * R + R; e += blockDim.x) {
        float s = 0.f;
        if (e < R * R) {
            const int i = e / R, j = e % R;
            for (int64_t row = r0; row < r1; row++) s = fmaf(phi(k[row * W + h * R + i]), v[row * W + h * R + j], s);
        } else {
            const int i = e - R * R;
            for (int64_t row = r0; row < r1; row++) s += phi(k[row * W + h * R + i]);
        }
        out[e] = s;
    }
}

// Adds the range partials: a workgroup of 16 wavefronts owns 64 consecutive outputs,
// wavefront w adds ranges w, w+16, ... and the 16 sums are added in wavefront order.
// Writes S and z into the workspace (and s_out / z_out if given).
__global__ __launch_bounds__(1024) void stats_reduce(int nb, int32_t H, int32_t R, const float* __restrict__ part,
                                                     float* __restrict__ s, float* __restrict__ z,
                                                     float* __restrict__ s_out, float* __restrict__ z_out) {
    __shared__ float sm[16][64];
    const int per = R * R + R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t x = (int64_t)blockIdx.x * 64 + lane;
    const int64_t tot = (int64_t)H * per;
    const int h = (int)(x / per), e = (int)(x % per);
    float a = 0.f;
    if (x < tot)
        for (int b = wave; b < nb; b += 16) a += part[((int64_t)b * H + h) * per + e];
    sm[wave][lane] = a;
    __syncthreads();
    if (wave != 0 || x >= tot) return;
    float t = 0.f;
    for (int w = 0; w < 16; w++) t += sm[w][lane];
    if (e < R * R) {
        s[(int64_t)h * R * R + e] = t;
        if (s_out) s_out[(int64_t)h * R * R + e] = t;
    } else {
        z[(int64_t)h * R + e - R * R] = t;
        if (z_out) z_out[(int64_t)h * R + e - R * R] = t;
    }
}

// ---- G = phi(Q) S / (phi(Q) z + eps), matrix-core path.  One wavefront per head (up to
// 16 per workgroup; the workgroup's wavefronts read the same rows), looping over 16-row
// tiles.  The contraction index is permuted so that in MFMA step t the lane group
// gq = lane/16 supplies k = gq*(R/4) + t: each lane's A operands over the R/4 steps are
// then R/4 consecutive elements of its row (16-byte loads), and its B operands S[k][j] are
// held in registers for the whole loop.
template <int TR>
__global__ __launch_bounds__(1024) void apply_mfma(int32_t n, int32_t H, float eps, const float* __restrict__ q,
                                                   const float* __restrict__ s, const float* __restrict__ z,
                                                   float* __restrict__ g) {
    constexpr int R = TR * 16;
    constexpr int KQ = R / 4;  // MFMA steps per row tile
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int64_t W = (int64_t)H * R;
    const int64_t tiles = ((int64_t)n + 15) / 16;
    for (int h = wave; h < H; h += nw) {
        float sreg[KQ][TR], zreg[KQ];
        // output columns are permuted too: MFMA tile j, position li <-> column TR*li + j, so
        // each lane ends with TR consecutive outputs of a row (one vector store)
#pragma unroll
        for (int t = 0; t < KQ; t++) {
            const int kk = gq * KQ + t;
            zreg[t] = z[(int64_t)h * R + kk];
#pragma unroll
            for (int j = 0; j < TR; j++) sreg[t][j] = s[((int64_t)h * R + kk) * R + TR * li + j];
        }
        for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
            const int64_t row = tile * 16 + li;
            float a[KQ];
            if (row < n) {
                const float4* qp = reinterpret_cast<const float4*>(q + row * W + h * R + gq * KQ);
#pragma unroll
                for (int c = 0; c < KQ / 4; c++) {
                    const float4 t4 = qp[c];
                    a[4 * c + 0] = phi(t4.x);
                    a[4 * c + 1] = phi(t4.y);
                    a[4 * c + 2] = phi(t4.z);
                    a[4 * c + 3] = phi(t4.w);
                }
            } else {
#pragma unroll
                for (int t = 0; t < KQ; t++) a[t] = 0.f;
            }
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < KQ; t++) d = fmaf(a[t], zreg[t], d);
            d += __shfl_xor(d, 16, 64);
            d += __shfl_xor(d, 32, 64);  // every lane li now holds the dot for row tile*16 + li
            v4f acc[TR];
#pragma unroll
            for (int j = 0; j < TR; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KQ; t++)
#pragma unroll
                for (int j = 0; j < TR; j++) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], sreg[t][j], acc[j], 0, 0, 0);
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int rr = gq * 4 + q4;  // output row of this lane within the tile
                const float inv = 1.0f / (__shfl(d, rr, 64) + eps);
                const int64_t orow = tile * 16 + rr;
                if (orow < n) {
                    float o[TR];
#pragma unroll
                    for (int j = 0; j < TR; j++) o[j] = acc[j][q4] * inv;
                    store_n<TR>(g + orow * W + h * R + TR * li, o);
                }
            }
        }
    }
}

// ---- G, scalar path.
__global__ void apply_scalar(int32_t n, int32_t H, int32_t R, float eps, const float* __restrict__ q,
                             const float* __restrict__ s, const float* __restrict__ z, float* __restrict__ g) {
    const int64_t W = (int64_t)H * R;
    for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < (int64_t)n * W;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = x / W;
        const int h = (int)((x % W) / R), j = (int)(x % R);
        const float* qr = q + row * W + h * R;
        float num = 0.f, d = 0.f;
        for (int c = 0; c < R; c++) {
            const float p = phi(qr[c]);
            num = fmaf(p, s[((int64_t)h * R + c) * R + j], num);
            d = fmaf(p, z[(int64_t)h * R + c], d);
        }
        g[x] = num / (d + eps);
    }
}

// ======================================================================== backward
// Gradients of sum(G * dG) for the branch above, per head, with S and z given:
//   num_i = phi(q_i)^T S, den_i = phi(q_i) . z + eps, G_i = num_i / den_i,
//   dnum_i = dG_i / den_i, dden_i = -(dG_i . G_i) / den_i,
//   dphi(q_i) = S dnum_i + z dden_i,   dS = sum_i phi(q_i) dnum_i^T,  dz = sum_i phi(q_i) dden_i,
//   dphi(k_j) = dS v_j + dz,           dv_j = dS^T phi(k_j),
// with phi'(x) = 1 for x > 0 and e^x otherwise.  dq, dk, dv are accumulated (+=).

__device__ __forceinline__ float dphi(float x, float p) { return x > 0.f ? 1.f : p; }

template <int N>
__device__ __forceinline__ void lds_load_n(const float* p, float* out) {
    if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        out[0] = t.x; out[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = p[i];
    }
}

// Loads the R x R matrix m[h] into LDS both as is (mr[c][j]) and transposed (mt[j][c]).
template <int R>
__device__ __forceinline__ void stage_both(const float* __restrict__ m, float* mr, float* mt) {
    for (int x = threadIdx.x; x < R * R; x += blockDim.x) {
        const float val = m[x];
        mr[x] = val;
        mt[(x % R) * R + x / R] = val;
    }
}

// ---- pass over the query rows, matrix-core path.  grid (nb, H), 4 wavefronts per
// workgroup, all on head blockIdx.y; the workgroup owns one node range (a multiple of 16
// rows) and its wavefronts take its 16-row tiles in turn.  Per tile, with the lane layout
// of apply_mfma (lane group gq = lane/16 owns the KQ consecutive features gq*KQ .. of the
// row li = lane%16):
//   1. num^T = S^T phi(Q)^T: A = S read from LDS, B = phi(q) of the lane's own row, so the
//      output lands with row li in lane li and columns gq*KQ + (q4*TR + jt) in group gq;
//   2. dphi(Q)^T = S dnum^T: A = S^T from LDS, B = the lane's own dnum;
//   3. dS += phi(Q)^T dnum: the tile's phi(q) and dnum go through LDS to put rows on the
//      contraction axis.
// The wavefronts' dS, dz sums are added in wavefront order and written as the range's
// partial (same layout as the statistics partials).
template <int TR>
__global__ __launch_bounds__(256) void dq_mfma(int32_t n, int32_t H, int32_t rows_per, float eps,
                                               const float* __restrict__ q, const float* __restrict__ s,
                                               const float* __restrict__ z, const float* __restrict__ dg,
                                               float* __restrict__ dq, float* __restrict__ part) {
    constexpr int R = TR * 16, KQ = R / 4;
    __shared__ float sl[R * R], st[R * R];
    __shared__ float pq[4][16 * R], dn_l[4][16 * R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per;
    const int64_t r1 = r0 + rows_per < n ? r0 + rows_per : n;
    stage_both<R>(s + (int64_t)h * R * R, sl, st);
    float zreg[KQ];
#pragma unroll
    for (int t = 0; t < KQ; t++) zreg[t] = z[(int64_t)h * R + gq * KQ + t];
    __syncthreads();

    v4f dsacc[TR][TR];
    float dzacc[KQ];
#pragma unroll
    for (int i = 0; i < TR; i++)
#pragma unroll
        for (int j = 0; j < TR; j++) dsacc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KQ; t++) dzacc[t] = 0.f;

    const int64_t ntile = r1 > r0 ? (r1 - r0 + 15) / 16 : 0;
    const int64_t iters = (ntile + 3) / 4;  // the same for every wavefront (block barriers below)
    for (int64_t it = 0; it < iters; it++) {
        const int64_t tl = it * 4 + wave;
        const int64_t row = r0 + tl * 16 + li;
        const bool valid = tl < ntile && row < r1;
        const int64_t off = row * W + h * R + gq * KQ;
        float qr[KQ], a[KQ], dgl[KQ];
        if (valid) {
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
                const float4 t4 = *reinterpret_cast<const float4*>(q + off + 4 * c);
                const float4 g4 = *reinterpret_cast<const float4*>(dg + off + 4 * c);
                qr[4 * c + 0] = t4.x; qr[4 * c + 1] = t4.y; qr[4 * c + 2] = t4.z; qr[4 * c + 3] = t4.w;
                dgl[4 * c + 0] = g4.x; dgl[4 * c + 1] = g4.y; dgl[4 * c + 2] = g4.z; dgl[4 * c + 3] = g4.w;
            }
#pragma unroll
            for (int t = 0; t < KQ; t++) a[t] = phi(qr[t]);
        } else {
#pragma unroll
            for (int t = 0; t < KQ; t++) qr[t] = a[t] = dgl[t] = 0.f;
        }
        float d = 0.f;
#pragma unroll
        for (int t = 0; t < KQ; t++) d = fmaf(a[t], zreg[t], d);
        d += __shfl_xor(d, 16, 64);
        d += __shfl_xor(d, 32, 64);
        const float inv = 1.0f / (d + eps);
        // 1. num^T
        v4f acc1[TR];
#pragma unroll
        for (int j = 0; j < TR; j++) acc1[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KQ; t++) {
            float sa[TR];
            lds_load_n<TR>(sl + (gq * KQ + t) * R + TR * li, sa);
#pragma unroll
            for (int j = 0; j < TR; j++) acc1[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[j], a[t], acc1[j], 0, 0, 0);
        }
        // acc1[jt][q4] = num[row li][gq*KQ + q4*TR + jt]
        float dn[KQ];
        float dd = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
#pragma unroll
            for (int j = 0; j < TR; j++) {
                const int idx = q4 * TR + j;
                dd = fmaf(dgl[idx], acc1[j][q4] * inv, dd);
                dn[idx] = dgl[idx] * inv;
            }
        dd += __shfl_xor(dd, 16, 64);
        dd += __shfl_xor(dd, 32, 64);
        const float dden = -dd * inv;
        // 2. dphi(Q)^T
        v4f acc2[TR];
#pragma unroll
        for (int j = 0; j < TR; j++) acc2[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KQ; t++) {
            float sa[TR];
            lds_load_n<TR>(st + (gq * KQ + t) * R + TR * li, sa);
#pragma unroll
            for (int c = 0; c < TR; c++) acc2[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[c], dn[t], acc2[c], 0, 0, 0);
        }
        // acc2[ct][q4] = (S dnum)[row li][gq*KQ + q4*TR + ct]
        if (valid) {
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
                float4* p = reinterpret_cast<float4*>(dq + off + 4 * c);
                float4 o = *p;
                float u[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int idx = 4 * c + e;
                    const float g = acc2[idx % TR][idx / TR] + zreg[idx] * dden;
                    u[e] = g * dphi(qr[idx], a[idx]);
                }
                o.x += u[0]; o.y += u[1]; o.z += u[2]; o.w += u[3];
                *p = o;
            }
        }
#pragma unroll
        for (int t = 0; t < KQ; t++) dzacc[t] = fmaf(a[t], dden, dzacc[t]);
        // 3. dS += phi(Q)^T dnum, rows moved onto the contraction axis through LDS
        float* pw = pq[wave];
        float* dw = dn_l[wave];
#pragma unroll
        for (int c = 0; c < KQ / 4; c++) {
            *reinterpret_cast<float4*>(pw + li * R + gq * KQ + 4 * c) =
                make_float4(a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]);
            *reinterpret_cast<float4*>(dw + li * R + gq * KQ + 4 * c) =
                make_float4(dn[4 * c], dn[4 * c + 1], dn[4 * c + 2], dn[4 * c + 3]);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; u++) {
            float pa[TR], pb[TR];
            lds_load_n<TR>(pw + (4 * u + gq) * R + TR * li, pa);
            lds_load_n<TR>(dw + (4 * u + gq) * R + TR * li, pb);
#pragma unroll
            for (int i = 0; i < TR; i++)
#pragma unroll
                for (int j = 0; j < TR; j++)
                    dsacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[i], pb[j], dsacc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // dz over the 16 rows of the lane group
#pragma unroll
    for (int t = 0; t < KQ; t++) {
        float v = dzacc[t];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        dzacc[t] = v;
    }
    // wavefronts add into sl (R*R) + st (first R) in wavefront order; each element has one owner lane
    float* buf = sl;
    float* zbuf = st;
    for (int w = 0; w < 4; w++) {
        if (wave == w) {
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
#pragma unroll
                for (int i = 0; i < TR; i++)
#pragma unroll
                    for (int j = 0; j < TR; j++) {
                        const int e = (TR * (gq * 4 + q4) + i) * R + TR * li + j;
                        buf[e] = (w == 0 ? 0.f : buf[e]) + dsacc[i][j][q4];
                    }
            if (li == 0) {
#pragma unroll
                for (int t = 0; t < KQ; t++) zbuf[gq * KQ + t] = (w == 0 ? 0.f : zbuf[gq * KQ + t]) + dzacc[t];
            }
        }
        __syncthreads();
    }
    float* out = part + ((int64_t)blockIdx.x * H + h) * (R * R + R);
    for (int x = threadIdx.x; x < R * R + R; x += blockDim.x) out[x] = x < R * R ? buf[x] : zbuf[x - R * R];
}

// ---- pass over the key rows, matrix-core path.  grid (blocks, H), 4 wavefronts per
// workgroup on head blockIdx.y, 16-row tiles strided over the grid.  dS and dS^T sit in LDS:
//   dphi(K)^T = dS V^T: A = dS^T rows, B = the lane's own v;
//   dV^T = dS^T phi(K)^T: A = dS rows, B = the lane's own phi(k).
template <int TR>
__global__ __launch_bounds__(256) void dkv_mfma(int32_t n, int32_t H, const float* __restrict__ k,
                                                const float* __restrict__ v, const float* __restrict__ ds,
                                                const float* __restrict__ dz, float* __restrict__ dk,
                                                float* __restrict__ dv) {
    constexpr int R = TR * 16, KQ = R / 4;
    __shared__ float sl[R * R], st[R * R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    stage_both<R>(ds + (int64_t)h * R * R, sl, st);
    float zreg[KQ];
#pragma unroll
    for (int t = 0; t < KQ; t++) zreg[t] = dz[(int64_t)h * R + gq * KQ + t];
    __syncthreads();
    const int64_t tiles = ((int64_t)n + 15) / 16;
    for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < tiles; tile += (int64_t)gridDim.x * 4) {
        const int64_t row = tile * 16 + li;
        const bool valid = row < n;
        const int64_t off = row * W + h * R + gq * KQ;
        float kr[KQ], pk[KQ], vv[KQ];
        if (valid) {
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
                const float4 k4 = *reinterpret_cast<const float4*>(k + off + 4 * c);
                const float4 v4 = *reinterpret_cast<const float4*>(v + off + 4 * c);
                kr[4 * c + 0] = k4.x; kr[4 * c + 1] = k4.y; kr[4 * c + 2] = k4.z; kr[4 * c + 3] = k4.w;
                vv[4 * c + 0] = v4.x; vv[4 * c + 1] = v4.y; vv[4 * c + 2] = v4.z; vv[4 * c + 3] = v4.w;
            }
#pragma unroll
            for (int t = 0; t < KQ; t++) pk[t] = phi(kr[t]);
        } else {
#pragma unroll
            for (int t = 0; t < KQ; t++) kr[t] = pk[t] = vv[t] = 0.f;
        }
        v4f ak[TR], av[TR];
#pragma unroll
        for (int j = 0; j < TR; j++) ak[j] = av[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KQ; t++) {
            float sa[TR], sb[TR];
            lds_load_n<TR>(st + (gq * KQ + t) * R + TR * li, sa);
            lds_load_n<TR>(sl + (gq * KQ + t) * R + TR * li, sb);
#pragma unroll
            for (int j = 0; j < TR; j++) {
                ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[j], vv[t], ak[j], 0, 0, 0);
                av[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sb[j], pk[t], av[j], 0, 0, 0);
            }
        }
        // ak[ct][q4] = (dS v)[row li][gq*KQ + q4*TR + ct]; av likewise for dS^T phi(k)
        if (valid) {
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
                float4* pk4 = reinterpret_cast<float4*>(dk + off + 4 * c);
                float4* pv4 = reinterpret_cast<float4*>(dv + off + 4 * c);
                float4 ok = *pk4, ov = *pv4;
                float uk[4], uv[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int idx = 4 * c + e;
                    uk[e] = (ak[idx % TR][idx / TR] + zreg[idx]) * dphi(kr[idx], pk[idx]);
                    uv[e] = av[idx % TR][idx / TR];
                }
                ok.x += uk[0]; ok.y += uk[1]; ok.z += uk[2]; ok.w += uk[3];
                ov.x += uv[0]; ov.y += uv[1]; ov.z += uv[2]; ov.w += uv[3];
                *pk4 = ok;
                *pv4 = ov;
            }
        }
    }
}

// ---- scalar paths (any r <= 64): one wavefront per row and head, lane c <-> feature c.
// grid (nb, H), 4 wavefronts per workgroup; the range's dS, dz partial as above.
__global__ __launch_bounds__(256) void dq_scalar(int32_t n, int32_t H, int32_t R, int32_t rows_per, float eps,
                                                 const float* __restrict__ q, const float* __restrict__ s,
                                                 const float* __restrict__ z, const float* __restrict__ dg,
                                                 float* __restrict__ dq, float* __restrict__ part) {
    __shared__ float buf[64 * 64 + 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per;
    const int64_t r1 = r0 + rows_per < n ? r0 + rows_per : n;
    const float* sh = s + (int64_t)h * R * R;
    const bool on = lane < R;
    const float zc = on ? z[(int64_t)h * R + lane] : 0.f;
    float acc[64];  // acc[c] = dS[c][lane]
#pragma unroll
    for (int c = 0; c < 64; c++) acc[c] = 0.f;
    float dzacc = 0.f;
    for (int64_t row = r0 + wave; row < r1; row += 4) {
        const int64_t off = row * W + h * R + lane;
        const float qc = on ? q[off] : 0.f;
        const float pc = on ? phi(qc) : 0.f;
        float d = pc * zc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) d += __shfl_xor(d, o, 64);
        const float inv = 1.0f / (d + eps);
        float num = 0.f;
        for (int c = 0; c < R; c++) num = fmaf(__shfl(pc, c, 64), on ? sh[c * R + lane] : 0.f, num);
        const float dgj = on ? dg[off] : 0.f;
        float dd = dgj * (num * inv);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) dd += __shfl_xor(dd, o, 64);
        const float dden = -dd * inv;
        const float dnj = dgj * inv;
        float dp = 0.f;
        for (int j = 0; j < R; j++) dp = fmaf(on ? sh[lane * R + j] : 0.f, __shfl(dnj, j, 64), dp);
        if (on) dq[off] += (dp + zc * dden) * dphi(qc, pc);
#pragma unroll
        for (int c = 0; c < 64; c++)
            if (c < R) acc[c] = fmaf(__shfl(pc, c, 64), dnj, acc[c]);
        dzacc = fmaf(pc, dden, dzacc);
    }
    for (int w = 0; w < 4; w++) {
        if (wave == w && on) {
#pragma unroll
            for (int c = 0; c < 64; c++)
                if (c < R) buf[c * R + lane] = (w == 0 ? 0.f : buf[c * R + lane]) + acc[c];
            buf[R * R + lane] = (w == 0 ? 0.f : buf[R * R + lane]) + dzacc;
        }
        __syncthreads();
    }
    float* out = part + ((int64_t)blockIdx.x * H + h) * (R * R + R);
    for (int x = threadIdx.x; x < R * R + R; x += blockDim.x) out[x] = buf[x];
}

__global__ __launch_bounds__(256) void dkv_scalar(int32_t n, int32_t H, int32_t R, const float* __restrict__ k,
                                                  const float* __restrict__ v, const float* __restrict__ ds,
                                                  const float* __restrict__ dz, float* __restrict__ dk,
                                                  float* __restrict__ dv) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const float* sh = ds + (int64_t)h * R * R;
    const bool on = lane < R;
    const float zc = on ? dz[(int64_t)h * R + lane] : 0.f;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < n; row += (int64_t)gridDim.x * 4) {
        const int64_t off = row * W + h * R + lane;
        const float kc = on ? k[off] : 0.f, vc = on ? v[off] : 0.f;
        const float pc = on ? phi(kc) : 0.f;
        float a = 0.f, b = 0.f;
        for (int j = 0; j < R; j++) a = fmaf(on ? sh[lane * R + j] : 0.f, __shfl(vc, j, 64), a);
        for (int c = 0; c < R; c++) b = fmaf(on ? sh[c * R + lane] : 0.f, __shfl(pc, c, 64), b);
        if (on) {
            dk[off] += (a + zc) * dphi(kc, pc);
            dv[off] += b;
        }
    }
}

struct GlWs {
    float* part;
    float* s;
    float* z;
    size_t bytes;
};

GlWs carve_gl(void* ws, int32_t n, int32_t H, int32_t R) {
    const int nb = row_ranges(n);
    Carver c(ws);
    GlWs w;
    w.part = c.take<float>((size_t)nb * H * (R * R + R));
    w.s = c.take<float>((size_t)H * R * R);
    w.z = c.take<float>((size_t)H * R);
    w.bytes = c.bytes();
    return w;
}

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" size_t gga_global_linear_workspace(int32_t n, int32_t heads, int32_t r) {
    if (n < 0 || heads < 1 || r < 1) return 0;
    return carve_gl(nullptr, n, heads, r).bytes;
}

extern "C" int gga_global_linear_fwd(int32_t n, int32_t heads, int32_t r, const float* q, const float* k,
                                     const float* v, float eps, float* s_out, float* z_out, float* g_out, void* ws,
                                     size_t ws_bytes, void* stream) {
    if (n < 0 || heads < 1 || r < 1) return GGA_EINVAL;
    if (r > 1024) return GGA_EUNSUPPORTED;
    if (n > 0 && (!q || !k || !v || !g_out)) return GGA_EINVAL;
    const GlWs need = carve_gl(nullptr, n, heads, r);
    if (ws_bytes < need.bytes || !ws) return GGA_EWORKSPACE;
    const GlWs w = carve_gl(ws, n, heads, r);
    hipStream_t s = as_stream(stream);
    const int nb = row_ranges(n);
    const int32_t rows_per = (int32_t)((((int64_t)n + nb - 1) / nb + 15) / 16 * 16);
    const bool mfma = r % 16 == 0 && r <= 64 && aligned16(q) && aligned16(k) && aligned16(v) && aligned16(g_out);
    const int wpb = heads < 16 ? heads : 16;  // wavefronts (heads) per workgroup
    if (n > 0) {
        if (mfma) {
            const unsigned grid = (unsigned)nb, threads = 64u * wpb;
            switch (r / 16) {
                case 1: stats_mfma<1><<<grid, threads, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
                case 2: stats_mfma<2><<<grid, threads, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
                case 3: stats_mfma<3><<<grid, threads, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
                default: stats_mfma<4><<<grid, threads, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
            }
        } else {
            stats_scalar<<<dim3((unsigned)nb, (unsigned)heads), 256, 0, s>>>(n, heads, r, rows_per, k, v, w.part);
        }
    } else {
        fill_f32(w.part, (int64_t)nb * heads * (r * r + r), 0.f, s);
    }
    const int64_t tot = (int64_t)heads * (r * r + r);
    stats_reduce<<<(unsigned)((tot + 63) / 64), 1024, 0, s>>>(nb, heads, r, w.part, w.s, w.z, s_out, z_out);
    if (n > 0) {
        if (mfma) {
            int64_t tiles = ((int64_t)n + 15) / 16;
            const unsigned grid = (unsigned)(tiles < 2048 ? tiles : 2048), threads = 64u * wpb;
            switch (r / 16) {
                case 1: apply_mfma<1><<<grid, threads, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
                case 2: apply_mfma<2><<<grid, threads, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
                case 3: apply_mfma<3><<<grid, threads, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
                default: apply_mfma<4><<<grid, threads, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
            }
        } else {
            int64_t blocks = ((int64_t)n * heads * r + 255) / 256;
            if (blocks > 65536) blocks = 65536;
            apply_scalar<<<(unsigned)blocks, 256, 0, s>>>(n, heads, r, eps, q, w.s, w.z, g_out);
        }
    }
    return launch_status();
}

extern "C" size_t gga_global_linear_bwd_workspace(int32_t n, int32_t heads, int32_t r) {
    if (n < 0 || heads < 1 || r < 1) return 0;
    return carve_gl(nullptr, n, heads, r).bytes;
}

extern "C" int gga_global_linear_bwd(int32_t n, int32_t heads, int32_t r, const float* q, const float* k,
                                     const float* v, float eps, const float* s_in, const float* z_in, const float* d_g,
                                     float* d_q, float* d_k, float* d_v, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || heads < 1 || r < 1) return GGA_EINVAL;
    if (r > 64) return GGA_EUNSUPPORTED;
    if (heads > 65535) return GGA_ERANGE;
    if (n == 0) return GGA_OK;
    if (!q || !k || !v || !s_in || !z_in || !d_g || !d_q || !d_k || !d_v) return GGA_EINVAL;
    const GlWs need = carve_gl(nullptr, n, heads, r);
    if (ws_bytes < need.bytes || !ws) return GGA_EWORKSPACE;
    const GlWs w = carve_gl(ws, n, heads, r);
    hipStream_t s = as_stream(stream);
    const int nb = row_ranges(n);
    const int32_t rows_per = (int32_t)((((int64_t)n + nb - 1) / nb + 15) / 16 * 16);
    const bool mfma = r % 16 == 0 && aligned16(q) && aligned16(k) && aligned16(v) && aligned16(d_g) &&
                      aligned16(d_q) && aligned16(d_k) && aligned16(d_v);
    const dim3 ga((unsigned)nb, (unsigned)heads);
    if (mfma) {
        switch (r / 16) {
            case 1: dq_mfma<1><<<ga, 256, 0, s>>>(n, heads, rows_per, eps, q, s_in, z_in, d_g, d_q, w.part); break;
            case 2: dq_mfma<2><<<ga, 256, 0, s>>>(n, heads, rows_per, eps, q, s_in, z_in, d_g, d_q, w.part); break;
            case 3: dq_mfma<3><<<ga, 256, 0, s>>>(n, heads, rows_per, eps, q, s_in, z_in, d_g, d_q, w.part); break;
            default: dq_mfma<4><<<ga, 256, 0, s>>>(n, heads, rows_per, eps, q, s_in, z_in, d_g, d_q, w.part); break;
        }
    } else {
        dq_scalar<<<ga, 256, 0, s>>>(n, heads, r, rows_per, eps, q, s_in, z_in, d_g, d_q, w.part);
    }
    const int64_t tot = (int64_t)heads * (r * r + r);
    stats_reduce<<<(unsigned)((tot + 63) / 64), 1024, 0, s>>>(nb, heads, r, w.part, w.s, w.z, nullptr, nullptr);
    const int64_t tiles = ((int64_t)n + 15) / 16;
    if (mfma) {
        int64_t blocks = (tiles + 3) / 4;
        if (blocks > 1024) blocks = 1024;
        const dim3 gb((unsigned)blocks, (unsigned)heads);
        switch (r / 16) {
            case 1: dkv_mfma<1><<<gb, 256, 0, s>>>(n, heads, k, v, w.s, w.z, d_k, d_v); break;
            case 2: dkv_mfma<2><<<gb, 256, 0, s>>>(n, heads, k, v, w.s, w.z, d_k, d_v); break;
            case 3: dkv_mfma<3><<<gb, 256, 0, s>>>(n, heads, k, v, w.s, w.z, d_k, d_v); break;
            default: dkv_mfma<4><<<gb, 256, 0, s>>>(n, heads, k, v, w.s, w.z, d_k, d_v); break;
        }
    } else {
        int64_t blocks = ((int64_t)n + 3) / 4;
        if (blocks > 4096) blocks = 4096;
        dkv_scalar<<<dim3((unsigned)blocks, (unsigned)heads), 256, 0, s>>>(n, heads, r, k, v, w.s, w.z, d_k, d_v);
    }
    return launch_status();
}
