// Node gate, branch combination and residual LayerNorm of the gated local-global layer
// ("Gated Local-Global Graph Attention", Key formulas g_i and Y_i; Implementation notes
// item 2, LayerNorm(X + Wo(g*L + (1-g)*G))).  One wavefront per node row; the reductions
// over a row use a fixed butterfly order.
#include "common.hpp"

namespace gga {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// gate[i] = sigmoid(gate_logit[i]); y[i] = gate[i] l[i] + (1 - gate[i]) g[i]
__global__ __launch_bounds__(256) void gated_combine_kernel(int32_t n, const float* __restrict__ logit, int32_t width,
                                                            const float* __restrict__ l,
                                                            const float* __restrict__ gg, float* __restrict__ gate,
                                                            float* __restrict__ y, int vec) {
    const int lane = threadIdx.x & 63;
    const int64_t i = blockIdx.x * 4ll + (threadIdx.x >> 6);
    if (i >= n) return;
    const float gv = 1.0f / (1.0f + __expf(-logit[i]));
    if (gate && lane == 0) gate[i] = gv;
    const float hv = 1.0f - gv;
    if (vec) {
        const float4* lr = reinterpret_cast<const float4*>(l + i * width);
        const float4* gr = reinterpret_cast<const float4*>(gg + i * width);
        float4* yr = reinterpret_cast<float4*>(y + i * width);
        for (int j = lane; j < width / 4; j += 64) {
            const float4 a = lr[j], b = gr[j];
            yr[j] = make_float4(gv * a.x + hv * b.x, gv * a.y + hv * b.y, gv * a.z + hv * b.z, gv * a.w + hv * b.w);
        }
    } else {
        for (int j = lane; j < width; j += 64) y[i * width + j] = gv * l[i * width + j] + hv * gg[i * width + j];
    }
}

// out = gamma * (a - mean) / sqrt(var + eps) + beta with a = x + y; two passes over the row
// held in registers (up to 64 * 4 * NV elements), biased variance.
template <int NV>
__global__ __launch_bounds__(256) void add_layernorm_kernel(int32_t n, int32_t d, const float* __restrict__ x,
                                                            const float* __restrict__ y,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, float eps,
                                                            float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t i = blockIdx.x * 4ll + (threadIdx.x >> 6);
    if (i >= n) return;
    const int d4 = d / 4;
    const float4* xr = reinterpret_cast<const float4*>(x + i * d);
    const float4* yr = reinterpret_cast<const float4*>(y + i * d);
    float4 a[NV];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int j = lane + 64 * k;
        if (j < d4) {
            const float4 p = xr[j], q = yr[j];
            a[k] = make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w);
            s += (a[k].x + a[k].y) + (a[k].z + a[k].w);
        } else {
            a[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const float mean = wave_sum(s) / (float)d;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int j = lane + 64 * k;
        if (j < d4) {
            const float dx = a[k].x - mean, dy = a[k].y - mean, dz = a[k].z - mean, dw = a[k].w - mean;
            v += (dx * dx + dy * dy) + (dz * dz + dw * dw);
        }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(v) / (float)d + eps);
    const float4* gr = reinterpret_cast<const float4*>(gamma);
    const float4* br = reinterpret_cast<const float4*>(beta);
    float4* orow = reinterpret_cast<float4*>(out + i * d);
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int j = lane + 64 * k;
        if (j < d4) {
            const float4 gm = gr[j], bt = br[j];
            orow[j] = make_float4(gm.x * (a[k].x - mean) * rstd + bt.x, gm.y * (a[k].y - mean) * rstd + bt.y,
                                  gm.z * (a[k].z - mean) * rstd + bt.z, gm.w * (a[k].w - mean) * rstd + bt.w);
        }
    }
}

// Any width: three passes re-reading the row.
__global__ __launch_bounds__(256) void add_layernorm_generic(int32_t n, int32_t d, const float* __restrict__ x,
                                                             const float* __restrict__ y,
                                                             const float* __restrict__ gamma,
                                                             const float* __restrict__ beta, float eps,
                                                             float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t i = blockIdx.x * 4ll + (threadIdx.x >> 6);
    if (i >= n) return;
    float s = 0.f;
    for (int j = lane; j < d; j += 64) s += x[i * d + j] + y[i * d + j];
    const float mean = wave_sum(s) / (float)d;
    float v = 0.f;
    for (int j = lane; j < d; j += 64) {
        const float t = x[i * d + j] + y[i * d + j] - mean;
        v += t * t;
    }
    const float rstd = 1.0f / sqrtf(wave_sum(v) / (float)d + eps);
    for (int j = lane; j < d; j += 64) out[i * d + j] = gamma[j] * (x[i * d + j] + y[i * d + j] - mean) * rstd + beta[j];
}

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" int gga_gated_combine(int32_t n, int32_t width, const float* gate_logit, const float* l, const float* g,
                                 float* gate_out, float* y, void* stream) {
    if (n < 0 || width < 1) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!gate_logit || !l || !g || !y) return GGA_EINVAL;
    const int vec = (width % 4 == 0) && aligned16(l) && aligned16(g) && aligned16(y);
    gated_combine_kernel<<<(unsigned)(((int64_t)n + 3) / 4), 256, 0, as_stream(stream)>>>(n, gate_logit, width, l, g,
                                                                                           gate_out, y, vec);
    return launch_status();
}

extern "C" int gga_add_layernorm(int32_t n, int32_t d, const float* x, const float* y, const float* gamma,
                                 const float* beta, float eps, float* out, void* stream) {
    if (n < 0 || d < 1) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!x || !y || !gamma || !beta || !out) return GGA_EINVAL;
    hipStream_t s = as_stream(stream);
    const unsigned grid = (unsigned)(((int64_t)n + 3) / 4);
    const bool vec = d % 4 == 0 && aligned16(x) && aligned16(y) && aligned16(gamma) && aligned16(beta) &&
                     aligned16(out);
    if (vec && d <= 256)
        add_layernorm_kernel<1><<<grid, 256, 0, s>>>(n, d, x, y, gamma, beta, eps, out);
    else if (vec && d <= 1024)
        add_layernorm_kernel<4><<<grid, 256, 0, s>>>(n, d, x, y, gamma, beta, eps, out);
    else
        add_layernorm_generic<<<grid, 256, 0, s>>>(n, d, x, y, gamma, beta, eps, out);
    return launch_status();
}
