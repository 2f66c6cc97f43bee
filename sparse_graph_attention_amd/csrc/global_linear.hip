// Global linear-attention branch ("Gated Local-Global Graph Attention", Key formulas G_i,
// S, z; Implementation notes item 2, phi = elu + 1), per head h of width r:
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

int row_ranges(int32_t n) {
    int64_t nb = ((int64_t)n + 1023) / 1024;
    if (nb < 1) nb = 1;
    if (nb > 256) nb = 256;
    return (int)nb;
}

// ---- statistics, matrix-core path.  grid (nb, H); block: 4 wavefronts splitting the
// range's rows four ways, folded in wavefront order.
template <int TR>
__global__ __launch_bounds__(256) void stats_mfma(int32_t n, int32_t H, int32_t rows_per, const float* __restrict__ k,
                                                  const float* __restrict__ v, float* __restrict__ part) {
    constexpr int R = TR * 16;
    __shared__ float sm[3][64][TR * TR * 4 + TR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per;
    const int64_t r1 = r0 + rows_per < n ? r0 + rows_per : n;
    v4f acc[TR][TR];
    float zacc[TR];
#pragma unroll
    for (int i = 0; i < TR; i++) {
        zacc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < TR; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t base = r0 + wave * 4; base < r1; base += 16) {
        const int64_t row = base + (lane >> 4);
        const bool ok = row < r1;
        float a[TR], b[TR];
#pragma unroll
        for (int t = 0; t < TR; t++) {
            const int64_t o = row * W + h * R + t * 16 + (lane & 15);
            a[t] = ok ? phi(k[o]) : 0.f;
            b[t] = ok ? v[o] : 0.f;
            zacc[t] += a[t];
        }
#pragma unroll
        for (int i = 0; i < TR; i++)
#pragma unroll
            for (int j = 0; j < TR; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TR; t++) {
        zacc[t] += __shfl_xor(zacc[t], 16, 64);
        zacc[t] += __shfl_xor(zacc[t], 32, 64);
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < TR; i++)
#pragma unroll
            for (int j = 0; j < TR; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) sm[wave - 1][lane][(i * TR + j) * 4 + q] = acc[i][j][q];
#pragma unroll
        for (int t = 0; t < TR; t++) sm[wave - 1][lane][TR * TR * 4 + t] = zacc[t];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 0; w < 3; w++) {
#pragma unroll
        for (int i = 0; i < TR; i++)
#pragma unroll
            for (int j = 0; j < TR; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) acc[i][j][q] += sm[w][lane][(i * TR + j) * 4 + q];
#pragma unroll
        for (int t = 0; t < TR; t++) zacc[t] += sm[w][lane][TR * TR * 4 + t];
    }
    float* out = part + ((int64_t)blockIdx.x * H + h) * (R * R + R);
#pragma unroll
    for (int i = 0; i < TR; i++)
#pragma unroll
        for (int j = 0; j < TR; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int ii = i * 16 + (lane >> 4) * 4 + q, jj = j * 16 + (lane & 15);
                out[ii * R + jj] = acc[i][j][q];
            }
    if (lane < 16)
#pragma unroll
        for (int t = 0; t < TR; t++) out[R * R + t * 16 + lane] = zacc[t];
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

// Adds the range partials in range order: S and z into ws (and s_out / z_out if given).
__global__ void stats_reduce(int nb, int32_t H, int32_t R, const float* __restrict__ part, float* __restrict__ s,
                             float* __restrict__ z, float* __restrict__ s_out, float* __restrict__ z_out) {
    const int per = R * R + R;
    for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < (int64_t)H * per;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int h = (int)(x / per), e = (int)(x % per);
        float a = 0.f;
        for (int b = 0; b < nb; b++) a += part[((int64_t)b * H + h) * per + e];
        if (e < R * R) {
            s[(int64_t)h * R * R + e] = a;
            if (s_out) s_out[(int64_t)h * R * R + e] = a;
        } else {
            z[(int64_t)h * R + e - R * R] = a;
            if (z_out) z_out[(int64_t)h * R + e - R * R] = a;
        }
    }
}

// ---- G = phi(Q) S / (phi(Q) z + eps), matrix-core path.  grid (ceil(n/64), H): a block
// stages 64 rows of phi(q) and S[h] in LDS; wavefront w computes rows w*16 .. w*16+15.
template <int TR>
__global__ __launch_bounds__(256) void apply_mfma(int32_t n, int32_t H, float eps, const float* __restrict__ q,
                                                  const float* __restrict__ s, const float* __restrict__ z,
                                                  float* __restrict__ g) {
    constexpr int R = TR * 16;
    __shared__ float Qs[64][R + 1];
    __shared__ float Ss[R][R + 4];
    __shared__ float den[64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t n0 = (int64_t)blockIdx.x * 64;
    for (int e = threadIdx.x; e < R * R; e += 256) Ss[e / R][e % R] = s[(int64_t)h * R * R + e];
    for (int e = threadIdx.x; e < 64 * R; e += 256) {
        const int rr = e / R, c = e % R;
        const int64_t row = n0 + rr;
        Qs[rr][c] = row < n ? phi(q[row * W + h * R + c]) : 0.f;
    }
    __syncthreads();
    {
        const int rr = threadIdx.x >> 2, part = threadIdx.x & 3;
        float d = 0.f;
        for (int c = part; c < R; c += 4) d = fmaf(Qs[rr][c], z[(int64_t)h * R + c], d);
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        if (part == 0) den[rr] = d + eps;
    }
    __syncthreads();
    v4f acc[TR];
#pragma unroll
    for (int j = 0; j < TR; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k4 = 0; k4 < R / 4; k4++) {
        const int kk = k4 * 4 + (lane >> 4);
        const float a = Qs[wave * 16 + (lane & 15)][kk];
#pragma unroll
        for (int j = 0; j < TR; j++) {
            const float b = Ss[kk][j * 16 + (lane & 15)];
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
        const int rr = wave * 16 + (lane >> 4) * 4 + q4;
        const int64_t row = n0 + rr;
        if (row >= n) continue;
        const float inv = 1.0f / den[rr];
#pragma unroll
        for (int j = 0; j < TR; j++) g[row * W + h * R + j * 16 + (lane & 15)] = acc[j][q4] * inv;
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
    const bool mfma = r % 16 == 0 && r <= 64;
    if (n > 0) {
        const dim3 grid((unsigned)nb, (unsigned)heads);
        if (mfma) {
            switch (r / 16) {
                case 1: stats_mfma<1><<<grid, 256, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
                case 2: stats_mfma<2><<<grid, 256, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
                case 3: stats_mfma<3><<<grid, 256, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
                default: stats_mfma<4><<<grid, 256, 0, s>>>(n, heads, rows_per, k, v, w.part); break;
            }
        } else {
            stats_scalar<<<grid, 256, 0, s>>>(n, heads, r, rows_per, k, v, w.part);
        }
    } else {
        fill_f32(w.part, (int64_t)nb * heads * (r * r + r), 0.f, s);
    }
    const int64_t tot = (int64_t)heads * (r * r + r);
    stats_reduce<<<(unsigned)((tot + 255) / 256), 256, 0, s>>>(nb, heads, r, w.part, w.s, w.z, s_out, z_out);
    if (n > 0) {
        if (mfma) {
            const dim3 grid((unsigned)(((int64_t)n + 63) / 64), (unsigned)heads);
            switch (r / 16) {
                case 1: apply_mfma<1><<<grid, 256, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
                case 2: apply_mfma<2><<<grid, 256, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
                case 3: apply_mfma<3><<<grid, 256, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
                default: apply_mfma<4><<<grid, 256, 0, s>>>(n, heads, eps, q, w.s, w.z, g_out); break;
            }
        } else {
            int64_t blocks = ((int64_t)n * heads * r + 255) / 256;
            if (blocks > 65536) blocks = 65536;
            apply_scalar<<<(unsigned)blocks, 256, 0, s>>>(n, heads, r, eps, q, w.s, w.z, g_out);
        }
    }
    return launch_status();
}
