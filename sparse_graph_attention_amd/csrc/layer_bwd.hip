// Backward of the node gate, branch combination and residual LayerNorm of the gated
// local-global layer ("Gated Local-Global Graph Attention", Key formulas g_i and Y_i;
// Implementation notes item 2).  One wavefront per node row for the row-local gradients;
// the parameter gradients (sums over rows) go through fixed-order partials: a workgroup
// owns a fixed range of rows, each of its wavefronts adds its rows into a private LDS row
// in row order, the wavefronts' rows are added in wavefront order, and a second kernel
// adds the ranges in range order.  Ranges and wavefront counts depend only on the shape,
// so the results are bit-identical from run to run.
#include "common.hpp"

namespace gga {
namespace {

constexpr int kLdsLimitFloats = 16384;  // 64 KiB of accumulators per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Accumulator rows are `stride` floats apart (ncols rounded up to 4, for 16-byte accesses).
__host__ __device__ constexpr int acc_stride(int ncols) { return (ncols + 3) / 4 * 4; }

struct RowSplit {
    int nb;          // ranges (workgroups)
    int32_t per;     // rows per range
    int wpb;         // wavefronts per workgroup
};

// Ranges of at least 64 rows, at most 1024 of them; up to 16 wavefronts per workgroup (each
// walks its rows one after another, so more of them keep more rows in flight), fewer when
// their accumulator rows (ncols floats each) would pass 64 KiB.
RowSplit row_split(int32_t n, int ncols) {
    RowSplit r;
    int64_t nb = ((int64_t)n + 63) / 64;
    if (nb < 1) nb = 1;
    if (nb > 1024) nb = 1024;
    r.nb = (int)nb;
    r.per = (int32_t)(((int64_t)n + nb - 1) / nb);
    int w = kLdsLimitFloats / acc_stride(ncols > 0 ? ncols : 1);
    r.wpb = w > 16 ? 16 : w;
    return r;
}

__device__ __forceinline__ void zero_acc(float* acc, int total) {
    for (int i = threadIdx.x; i < total; i += blockDim.x) acc[i] = 0.f;
    __syncthreads();
}

// part[blockIdx.x][col] = sum over the workgroup's wavefronts (in order) of acc[w][col]
__device__ __forceinline__ void flush_acc(const float* acc, int ncols, int nw, float* __restrict__ part) {
    __syncthreads();
    const int stride = acc_stride(ncols);
    for (int c = threadIdx.x; c < ncols; c += blockDim.x) {
        float s = 0.f;
        for (int w = 0; w < nw; w++) s += acc[w * stride + c];
        part[(int64_t)blockIdx.x * ncols + c] = s;
    }
}

// ---- LayerNorm backward, row held in registers (d % 4 == 0, d <= 256 * NV, aligned).
// Lane owns float4 columns lane + 64 k.  acc row: [0, d) d_gamma, [d, 2d) d_beta.
template <int NV>
__global__ __launch_bounds__(1024) void ln_bwd_vec(int32_t n, int32_t d, int32_t per, const float* __restrict__ x,
                                                   const float* __restrict__ y, const float* __restrict__ gamma,
                                                   float eps, const float* __restrict__ d_out,
                                                   float* __restrict__ d_pre, float* __restrict__ part) {
    extern __shared__ float acc_lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int ncols = 2 * d, d4 = d / 4;
    zero_acc(acc_lds, nw * acc_stride(ncols));
    float* acc = acc_lds + wave * acc_stride(ncols);
    const int64_t r0 = (int64_t)blockIdx.x * per;
    const int64_t r1 = r0 + per < n ? r0 + per : n;
    const float4* gr = reinterpret_cast<const float4*>(gamma);
    for (int64_t i = r0 + wave; i < r1; i += nw) {
        const float4* xr = reinterpret_cast<const float4*>(x + i * d);
        const float4* yr = reinterpret_cast<const float4*>(y + i * d);
        const float4* dr = reinterpret_cast<const float4*>(d_out + i * d);
        float4 a[NV], go[NV];
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < NV; k++) {
            const int j = lane + 64 * k;
            if (j < d4) {
                const float4 p = xr[j], q = yr[j];
                a[k] = make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w);
                go[k] = dr[j];
                s += (a[k].x + a[k].y) + (a[k].z + a[k].w);
            } else {
                a[k] = go[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        const float mean = wave_sum(s) / (float)d;
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < NV; k++) {
            if (lane + 64 * k < d4) {
                a[k] = make_float4(a[k].x - mean, a[k].y - mean, a[k].z - mean, a[k].w - mean);
                v += (a[k].x * a[k].x + a[k].y * a[k].y) + (a[k].z * a[k].z + a[k].w * a[k].w);
            }
        }
        const float rstd = 1.0f / sqrtf(wave_sum(v) / (float)d + eps);
        // a <- xhat; s1 = sum g, s2 = sum g xhat with g = d_out gamma
        float s1 = 0.f, s2 = 0.f;
        float4 gg[NV];
#pragma unroll
        for (int k = 0; k < NV; k++) {
            const int j = lane + 64 * k;
            if (j < d4) {
                a[k] = make_float4(a[k].x * rstd, a[k].y * rstd, a[k].z * rstd, a[k].w * rstd);
                const float4 gm = gr[j];
                gg[k] = make_float4(go[k].x * gm.x, go[k].y * gm.y, go[k].z * gm.z, go[k].w * gm.w);
                s1 += (gg[k].x + gg[k].y) + (gg[k].z + gg[k].w);
                s2 += (gg[k].x * a[k].x + gg[k].y * a[k].y) + (gg[k].z * a[k].z + gg[k].w * a[k].w);
            } else {
                gg[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        const float m1 = wave_sum(s1) / (float)d, m2 = wave_sum(s2) / (float)d;
        float4* pr = reinterpret_cast<float4*>(d_pre + i * d);
#pragma unroll
        for (int k = 0; k < NV; k++) {
            const int j = lane + 64 * k;
            if (j < d4) {
                pr[j] = make_float4(rstd * (gg[k].x - m1 - a[k].x * m2), rstd * (gg[k].y - m1 - a[k].y * m2),
                                    rstd * (gg[k].z - m1 - a[k].z * m2), rstd * (gg[k].w - m1 - a[k].w * m2));
                float4* ag = reinterpret_cast<float4*>(acc + 4 * j);
                float4* ab = reinterpret_cast<float4*>(acc + d + 4 * j);
                float4 t = *ag;
                t.x = fmaf(go[k].x, a[k].x, t.x);
                t.y = fmaf(go[k].y, a[k].y, t.y);
                t.z = fmaf(go[k].z, a[k].z, t.z);
                t.w = fmaf(go[k].w, a[k].w, t.w);
                *ag = t;
                float4 b = *ab;
                b.x += go[k].x;
                b.y += go[k].y;
                b.z += go[k].z;
                b.w += go[k].w;
                *ab = b;
            }
        }
    }
    flush_acc(acc_lds, ncols, nw, part);
}

// ---- LayerNorm backward, any width: passes re-read the row (from cache).
__global__ __launch_bounds__(1024) void ln_bwd_generic(int32_t n, int32_t d, int32_t per, const float* __restrict__ x,
                                                       const float* __restrict__ y, const float* __restrict__ gamma,
                                                       float eps, const float* __restrict__ d_out,
                                                       float* __restrict__ d_pre, float* __restrict__ part) {
    extern __shared__ float acc_lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int ncols = 2 * d;
    zero_acc(acc_lds, nw * acc_stride(ncols));
    float* acc = acc_lds + wave * acc_stride(ncols);
    const int64_t r0 = (int64_t)blockIdx.x * per;
    const int64_t r1 = r0 + per < n ? r0 + per : n;
    for (int64_t i = r0 + wave; i < r1; i += nw) {
        const float* xr = x + i * d;
        const float* yr = y + i * d;
        const float* dr = d_out + i * d;
        float s = 0.f;
        for (int j = lane; j < d; j += 64) s += xr[j] + yr[j];
        const float mean = wave_sum(s) / (float)d;
        float v = 0.f;
        for (int j = lane; j < d; j += 64) {
            const float t = xr[j] + yr[j] - mean;
            v += t * t;
        }
        const float rstd = 1.0f / sqrtf(wave_sum(v) / (float)d + eps);
        float s1 = 0.f, s2 = 0.f;
        for (int j = lane; j < d; j += 64) {
            const float xh = (xr[j] + yr[j] - mean) * rstd, g = dr[j] * gamma[j];
            s1 += g;
            s2 += g * xh;
        }
        const float m1 = wave_sum(s1) / (float)d, m2 = wave_sum(s2) / (float)d;
        for (int j = lane; j < d; j += 64) {
            const float xh = (xr[j] + yr[j] - mean) * rstd, go = dr[j];
            d_pre[i * d + j] = rstd * (go * gamma[j] - m1 - xh * m2);
            acc[j] = fmaf(go, xh, acc[j]);
            acc[d + j] += go;
        }
    }
    flush_acc(acc_lds, ncols, nw, part);
}

// ---- gate and combination backward.  acc row: [0, d) d_w_g, [d] d_b_g.
// XOUT: write d_x_out = d_x_in + dt w_g^T; otherwise only the logit gradients dt (d_logit,
// when given) leave, and the caller adds dt w_g^T into dX elsewhere.
template <bool XOUT>
__global__ __launch_bounds__(1024) void combine_bwd_kernel(int32_t n, int32_t d, int32_t per, const float* __restrict__ x,
                                                           const float* __restrict__ w_g, float b_g, int32_t width,
                                                           const float* __restrict__ l, const float* __restrict__ gg,
                                                           const float* __restrict__ d_y, float* __restrict__ d_l,
                                                           float* __restrict__ d_g, const float* d_x_in,
                                                           float* d_x_out, float* __restrict__ d_logit,
                                                           float* __restrict__ part, int vec) {
    extern __shared__ float acc_lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int ncols = d + 1;
    zero_acc(acc_lds, nw * acc_stride(ncols));
    float* acc = acc_lds + wave * acc_stride(ncols);
    const int64_t r0 = (int64_t)blockIdx.x * per;
    const int64_t r1 = r0 + per < n ? r0 + per : n;
    for (int64_t i = r0 + wave; i < r1; i += nw) {
        // gate
        float t = 0.f;
        if (vec) {
            const float4* xr = reinterpret_cast<const float4*>(x + i * d);
            const float4* wr = reinterpret_cast<const float4*>(w_g);
            for (int j = lane; j < d / 4; j += 64) {
                const float4 a = xr[j], b = wr[j];
                t = fmaf(a.x, b.x, t);
                t = fmaf(a.y, b.y, t);
                t = fmaf(a.z, b.z, t);
                t = fmaf(a.w, b.w, t);
            }
        } else {
            for (int j = lane; j < d; j += 64) t = fmaf(x[i * d + j], w_g[j], t);
        }
        t = wave_sum(t) + b_g;
        const float gv = 1.0f / (1.0f + __expf(-t));
        const float hv = 1.0f - gv;
        // branch gradients and the gate's share
        float s = 0.f;
        if (vec) {
            const float4* lr = reinterpret_cast<const float4*>(l + i * width);
            const float4* gr = reinterpret_cast<const float4*>(gg + i * width);
            const float4* yr = reinterpret_cast<const float4*>(d_y + i * width);
            float4* dlr = reinterpret_cast<float4*>(d_l + i * width);
            float4* dgr = reinterpret_cast<float4*>(d_g + i * width);
            for (int j = lane; j < width / 4; j += 64) {
                const float4 a = lr[j], b = gr[j], dy = yr[j];
                dlr[j] = make_float4(gv * dy.x, gv * dy.y, gv * dy.z, gv * dy.w);
                dgr[j] = make_float4(hv * dy.x, hv * dy.y, hv * dy.z, hv * dy.w);
                s += (dy.x * (a.x - b.x) + dy.y * (a.y - b.y)) + (dy.z * (a.z - b.z) + dy.w * (a.w - b.w));
            }
        } else {
            for (int j = lane; j < width; j += 64) {
                const int64_t o = i * width + j;
                const float dy = d_y[o];
                d_l[o] = gv * dy;
                d_g[o] = hv * dy;
                s += dy * (l[o] - gg[o]);
            }
        }
        const float dt = wave_sum(s) * (gv * hv);
        if (d_logit && lane == 0) d_logit[i] = dt;
        // input gradient and the parameter partials
        if (vec) {
            const float4* xr = reinterpret_cast<const float4*>(x + i * d);
            const float4* wr = reinterpret_cast<const float4*>(w_g);
            for (int j = lane; j < d / 4; j += 64) {
                const float4 a = xr[j];
                if constexpr (XOUT) {
                    const float4 w = wr[j], p = reinterpret_cast<const float4*>(d_x_in + i * d)[j];
                    reinterpret_cast<float4*>(d_x_out + i * d)[j] =
                        make_float4(fmaf(dt, w.x, p.x), fmaf(dt, w.y, p.y), fmaf(dt, w.z, p.z), fmaf(dt, w.w, p.w));
                }
                float4* ap = reinterpret_cast<float4*>(acc + 4 * j);
                float4 c = *ap;
                c.x = fmaf(dt, a.x, c.x);
                c.y = fmaf(dt, a.y, c.y);
                c.z = fmaf(dt, a.z, c.z);
                c.w = fmaf(dt, a.w, c.w);
                *ap = c;
            }
        } else {
            for (int j = lane; j < d; j += 64) {
                const int64_t o = i * d + j;
                if constexpr (XOUT) d_x_out[o] = fmaf(dt, w_g[j], d_x_in[o]);
                acc[j] = fmaf(dt, x[o], acc[j]);
            }
        }
        if (lane == 0) acc[d] += dt;
    }
    flush_acc(acc_lds, ncols, nw, part);
}

// Adds the range partials part[nb][ncols] in range order: a workgroup of 16 wavefronts owns
// 64 columns, wavefront w adds ranges w, w+16, ... and the 16 sums are added in wavefront
// order.  Columns below `split` go to out0, the rest to out1.
__global__ __launch_bounds__(1024) void colsum_reduce(int nb, int ncols, const float* __restrict__ part, int split,
                                                      float* __restrict__ out0, float* __restrict__ out1) {
    __shared__ float sm[16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    float a = 0.f;
    if (c < ncols) {
        // eight of the wavefront's ranges are requested at a time and added in range order
        // (the same sums as one at a time)
        int b = wave;
        for (; b + 7 * 16 < nb; b += 8 * 16) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = part[(int64_t)(b + 16 * j) * ncols + c];
#pragma unroll
            for (int j = 0; j < 8; j++) a += v[j];
        }
        for (; b < nb; b += 16) a += part[(int64_t)b * ncols + c];
    }
    sm[wave][lane] = a;
    __syncthreads();
    if (wave != 0 || c >= ncols) return;
    float t = 0.f;
    for (int w = 0; w < 16; w++) t += sm[w][lane];
    if (c < split)
        out0[c] = t;
    else
        out1[c - split] = t;
}

size_t part_bytes(int32_t n, int ncols) {
    const RowSplit r = row_split(n, ncols);
    return align_up((size_t)r.nb * ncols * sizeof(float), 256);
}

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" size_t gga_add_layernorm_bwd_workspace(int32_t n, int32_t d) {
    if (n < 0 || d < 1) return 0;
    return part_bytes(n, 2 * d);
}

extern "C" int gga_add_layernorm_bwd(int32_t n, int32_t d, const float* x, const float* y, const float* gamma,
                                     float eps, const float* d_out, float* d_pre, float* d_gamma, float* d_beta,
                                     void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || d < 1) return GGA_EINVAL;
    if (!gamma || !d_gamma || !d_beta) return GGA_EINVAL;
    if (n > 0 && (!x || !y || !d_out || !d_pre)) return GGA_EINVAL;
    const int ncols = 2 * d;
    const RowSplit rs = row_split(n, ncols);
    if (rs.wpb < 1) return GGA_EUNSUPPORTED;
    const size_t need = part_bytes(n, ncols);
    if (ws_bytes < need || !ws) return GGA_EWORKSPACE;
    hipStream_t s = as_stream(stream);
    float* part = static_cast<float*>(ws);
    const unsigned threads = 64u * rs.wpb;
    const size_t lds = (size_t)rs.wpb * acc_stride(ncols) * sizeof(float);
    const bool vec = d % 4 == 0 && aligned16(x) && aligned16(y) && aligned16(gamma) && aligned16(d_out) &&
                     aligned16(d_pre);
    if (n == 0)
        fill_f32(part, (int64_t)rs.nb * ncols, 0.f, s);
    else if (vec && d <= 256)
        ln_bwd_vec<1><<<(unsigned)rs.nb, threads, lds, s>>>(n, d, rs.per, x, y, gamma, eps, d_out, d_pre, part);
    else if (vec && d <= 512)
        ln_bwd_vec<2><<<(unsigned)rs.nb, threads, lds, s>>>(n, d, rs.per, x, y, gamma, eps, d_out, d_pre, part);
    else if (vec && d <= 1024)
        ln_bwd_vec<4><<<(unsigned)rs.nb, threads, lds, s>>>(n, d, rs.per, x, y, gamma, eps, d_out, d_pre, part);
    else
        ln_bwd_generic<<<(unsigned)rs.nb, threads, lds, s>>>(n, d, rs.per, x, y, gamma, eps, d_out, d_pre, part);
    colsum_reduce<<<(unsigned)((ncols + 63) / 64), 1024, 0, s>>>(rs.nb, ncols, part, d, d_gamma, d_beta);
    return launch_status();
}

extern "C" size_t gga_gated_combine_bwd_workspace(int32_t n, int32_t d) {
    if (n < 0 || d < 1) return 0;
    return part_bytes(n, d + 1);
}

extern "C" int gga_gated_combine_bwd(int32_t n, int32_t d, const float* x, const float* w_g, float b_g, int32_t width,
                                     const float* l, const float* g_glob, const float* d_y, float* d_l, float* d_g,
                                     const float* d_x_in, float* d_x_out, float* d_logit, float* d_w_g, float* d_b_g,
                                     void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || d < 1 || width < 1) return GGA_EINVAL;
    if (!w_g || !d_w_g || !d_b_g) return GGA_EINVAL;
    // d_x_in and d_x_out come together; without them d_logit must be given (rows only)
    if (n > 0 && ((d_x_in == nullptr) != (d_x_out == nullptr) || (!d_x_out && !d_logit))) return GGA_EINVAL;
    if (n > 0 && (!x || !l || !g_glob || !d_y || !d_l || !d_g)) return GGA_EINVAL;
    const int ncols = d + 1;
    const RowSplit rs = row_split(n, ncols);
    if (rs.wpb < 1) return GGA_EUNSUPPORTED;
    const size_t need = part_bytes(n, ncols);
    if (ws_bytes < need || !ws) return GGA_EWORKSPACE;
    hipStream_t s = as_stream(stream);
    float* part = static_cast<float*>(ws);
    const int vec = (d % 4 == 0) && (width % 4 == 0) && aligned16(x) && aligned16(w_g) && aligned16(l) &&
                    aligned16(g_glob) && aligned16(d_y) && aligned16(d_l) && aligned16(d_g) && aligned16(d_x_in) &&
                    aligned16(d_x_out);
    if (n == 0)
        fill_f32(part, (int64_t)rs.nb * ncols, 0.f, s);
    else if (d_x_out)
        combine_bwd_kernel<true><<<(unsigned)rs.nb, 64u * rs.wpb, (size_t)rs.wpb * acc_stride(ncols) * sizeof(float),
                                   s>>>(n, d, rs.per, x, w_g, b_g, width, l, g_glob, d_y, d_l, d_g, d_x_in, d_x_out,
                                        d_logit, part, vec);
    else
        combine_bwd_kernel<false><<<(unsigned)rs.nb, 64u * rs.wpb, (size_t)rs.wpb * acc_stride(ncols) * sizeof(float),
                                    s>>>(n, d, rs.per, x, w_g, b_g, width, l, g_glob, d_y, d_l, d_g, nullptr, nullptr,
                                         d_logit, part, vec);
    colsum_reduce<<<(unsigned)((ncols + 63) / 64), 1024, 0, s>>>(rs.nb, ncols, part, d, d_w_g, d_b_g);
    return launch_status();
}
