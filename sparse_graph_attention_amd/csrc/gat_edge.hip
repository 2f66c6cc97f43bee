// Endpoint projection (Tinymesh "Sparse attention experiment", section "Endpoint
// projection") and the GAT node coefficients (section "Composition").
#include "common.hpp"

namespace gga {
namespace {

// out[e, :] = x[endpoint[e], :], copied in 16-byte units when rows allow it.
template <typename U>
__global__ void edge_gather(const U* __restrict__ x, const int32_t* __restrict__ endpoint, int64_t e, int32_t units,
                            U* __restrict__ out) {
    const int64_t total = e * units;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ed = i / units;
        const int32_t c = (int32_t)(i - ed * units);
        out[i] = x[(int64_t)endpoint[ed] * units + c];
    }
}

// dx[u, :] = sum over the CSR row u of d_edge[eid[p], :].  One wavefront per row; its
// 64/LW lane groups take interleaved edges and are added in a fixed butterfly order.
__global__ __launch_bounds__(256) void edge_scatter_sum(int32_t n, int32_t width, int32_t lw_log2,
                                                        const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ eid,
                                                        const float* __restrict__ d_edge, float* __restrict__ dx) {
    const int lane = threadIdx.x & 63;
    const int lw = 1 << lw_log2;
    const int G = 64 >> lw_log2;
    const int g = lane >> lw_log2, li = lane & (lw - 1);
    const int64_t u = blockIdx.x * 4ll + (threadIdx.x >> 6);
    if (u >= n) return;
    const int32_t beg = row_ptr[u], end = row_ptr[u + 1];
    for (int x0 = 0; x0 < width; x0 += lw) {
        const int x = x0 + li;
        float acc = 0.f;
        for (int64_t p = beg + g; p < end; p += G) {  // (64-bit: end may lie within G of INT32_MAX)
            const int64_t ed = eid[p];
            if (x < width) acc += d_edge[ed * width + x];
        }
        for (int o = lw; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
        if (g == 0 && x < width) dx[u * width + x] = acc;
    }
}

// s_src[n,h] = a_s[h,:] . hf[n,h,:],  s_dst[n,h] = a_t[h,:] . hf[n,h,:] (skipped when
// a_t is null: one coefficient per row, as for the edge term)
__global__ void coef_fwd(int64_t nh, int32_t heads, int32_t c, const float* __restrict__ hf,
                         const float* __restrict__ a_s, const float* __restrict__ a_t, float* __restrict__ s_src,
                         float* __restrict__ s_dst, int vec) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nh; i += (int64_t)gridDim.x * blockDim.x) {
        const int h = (int)(i % heads);
        const float* row = hf + i * c;
        float ss = 0.f, st = 0.f;
        if (vec) {  // c % 4 == 0, 16-byte aligned rows: the wavefront reads whole rows in 16-byte pieces
            for (int j = 0; j < c; j += 4) {
                const float4 v = *reinterpret_cast<const float4*>(row + j);
                const float* as = a_s + h * c + j;
                ss = fmaf(as[0], v.x, ss);
                ss = fmaf(as[1], v.y, ss);
                ss = fmaf(as[2], v.z, ss);
                ss = fmaf(as[3], v.w, ss);
                if (a_t) {
                    const float* at = a_t + h * c + j;
                    st = fmaf(at[0], v.x, st);
                    st = fmaf(at[1], v.y, st);
                    st = fmaf(at[2], v.z, st);
                    st = fmaf(at[3], v.w, st);
                }
            }
        } else {
            for (int j = 0; j < c; j++) {
                const float v = row[j];
                ss = fmaf(a_s[h * c + j], v, ss);
                if (a_t) st = fmaf(a_t[h * c + j], v, st);
            }
        }
        s_src[i] = ss;
        if (a_t) s_dst[i] = st;
    }
}

// Fixed split of the row axis for the coefficient gradients: ranges of about 64 rows (enough
// workgroups to keep every CU's loads in flight), at least 1 and at most 16384 of them (a
// function of n, so the order of the sums is too).
inline int coef_blocks(int64_t n) {
    int64_t b = (n + 63) / 64;
    if (b < 1) b = 1;
    if (b > 16384) b = 16384;
    return (int)b;
}

// d_hf = d_hf_attn + a_s d_s_src + a_t d_s_dst (elementwise), and per-block partial sums of
// d_s_src * hf and d_s_dst * hf over a fixed node range.  d_hf_attn may be null (zero); a_t
// and d_s_dst may be null (one coefficient per row).
__global__ __launch_bounds__(256) void coef_bwd_partial(int32_t n, int32_t heads, int32_t c,
                                                        const float* __restrict__ hf, const float* __restrict__ a_s,
                                                        const float* __restrict__ a_t,
                                                        const float* __restrict__ d_hf_attn,
                                                        const float* __restrict__ d_ss,
                                                        const float* __restrict__ d_sd, float* __restrict__ d_hf,
                                                        float* __restrict__ part) {
    const int W = heads * c;
    const int64_t rows_per = ((int64_t)n + gridDim.x - 1) / gridDim.x;
    const int64_t r0 = blockIdx.x * rows_per;
    const int64_t r1 = r0 + rows_per < n ? r0 + rows_per : n;
    __shared__ float sm[2][256];
    for (int x0 = 0; x0 < W; x0 += 256) {
        // threads cover (row group, element): 256 / we row groups
        const int we = (W - x0) < 256 ? (W - x0) : 256;
        const int groups = 256 / we;
        const int gi = threadIdx.x / we, x = x0 + threadIdx.x % we;
        float as_ = 0.f, at_ = 0.f;
        if (gi < groups) {
            const int h = x / c;
            const float ws = a_s[x], wt = a_t ? a_t[x] : 0.f;
            for (int64_t r = r0 + gi; r < r1; r += groups) {
                const int64_t i = r * W + x;
                const float v = hf[i];
                const float gs = d_ss[r * heads + h], gt = d_sd ? d_sd[r * heads + h] : 0.f;
                d_hf[i] = (d_hf_attn ? d_hf_attn[i] : 0.f) + ws * gs + wt * gt;
                as_ = fmaf(gs, v, as_);
                at_ = fmaf(gt, v, at_);
            }
        }
        // fold the row groups in order
        for (int k = 0; k < groups; k++) {
            __syncthreads();
            if (gi == k) {
                const int t = threadIdx.x % we;
                sm[0][t] = (k == 0 ? 0.f : sm[0][t]) + as_;
                sm[1][t] = (k == 0 ? 0.f : sm[1][t]) + at_;
            }
        }
        __syncthreads();
        if ((int)threadIdx.x < we) {
            part[((int64_t)blockIdx.x * 2 + 0) * W + x0 + threadIdx.x] = sm[0][threadIdx.x];
            part[((int64_t)blockIdx.x * 2 + 1) * W + x0 + threadIdx.x] = sm[1][threadIdx.x];
        }
        __syncthreads();
    }
}

// One workgroup per output: thread t adds ranges t, t+256, ... and the 256 sums are added
// by a fixed tree.
__global__ __launch_bounds__(256) void coef_bwd_reduce(int32_t W, int nb, const float* __restrict__ part,
                                                       float* __restrict__ d_a_s, float* __restrict__ d_a_t) {
    __shared__ float sm[256];
    const int x = blockIdx.x;
    const int which = x / W, y = x % W;
    if (which == 1 && !d_a_t) return;
    float a = 0.f;
    int b = threadIdx.x;
    for (; b + 7 * 256 < nb; b += 8 * 256) {  // eight ranges requested at a time, added in order
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = part[((int64_t)(b + 256 * j) * 2 + which) * W + y];
#pragma unroll
        for (int j = 0; j < 8; j++) a += v[j];
    }
    for (; b < nb; b += 256) a += part[((int64_t)b * 2 + which) * W + y];
    sm[threadIdx.x] = a;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) sm[threadIdx.x] += sm[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) (which == 0 ? d_a_s : d_a_t)[y] = sm[0];
}

// out[n, c] = (1/H) sum_h in[n, h, c] (heads averaged, in head order)
__global__ void head_mean_kernel(int64_t nc, int32_t heads, int32_t c, const float* __restrict__ in,
                                 float* __restrict__ out) {
    const float inv = 1.0f / (float)heads;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nc; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = i / c;
        const int j = (int)(i - n * c);
        const float* row = in + n * heads * c + j;
        float a = 0.f;
        for (int h = 0; h < heads; h++) a += row[(int64_t)h * c];
        out[i] = a * inv;
    }
}

// d_in[n, h, c] = d_out[n, c] / H
__global__ void head_mean_bwd_kernel(int64_t total, int32_t heads, int32_t c, const float* __restrict__ d_out,
                                     float* __restrict__ d_in) {
    const float inv = 1.0f / (float)heads;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = i / ((int64_t)heads * c);
        const int j = (int)(i % c);
        d_in[i] = d_out[n * c + j] * inv;
    }
}

int grid_for(int64_t n, int threads) {
    int64_t b = (n + threads - 1) / threads;
    if (b < 1) b = 1;
    if (b > 65536) b = 65536;
    return (int)b;
}

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" int gga_edge_values(int32_t n, int32_t width, int32_t dtype, const void* x, int64_t e,
                               const int32_t* endpoint, void* out, void* stream) {
    if (n < 0 || width < 1 || e < 0) return GGA_EINVAL;
    if (dtype != GGA_F32 && dtype != GGA_BF16) return GGA_EUNSUPPORTED;
    if (e == 0) return GGA_OK;
    if (!x || !endpoint || !out || n == 0) return GGA_EINVAL;
    const int esz = dtype == GGA_BF16 ? 2 : 4;
    const int64_t rb = (int64_t)width * esz;
    hipStream_t s = as_stream(stream);
    if (rb % 16 == 0 && aligned16(x) && aligned16(out)) {
        const int32_t units = (int32_t)(rb / 16);
        edge_gather<uint4><<<grid_for(e * units, 256), 256, 0, s>>>(static_cast<const uint4*>(x), endpoint, e, units,
                                                                     static_cast<uint4*>(out));
    } else if (esz == 4) {
        edge_gather<float><<<grid_for(e * width, 256), 256, 0, s>>>(static_cast<const float*>(x), endpoint, e, width,
                                                                     static_cast<float*>(out));
    } else {
        edge_gather<uint16_t><<<grid_for(e * width, 256), 256, 0, s>>>(static_cast<const uint16_t*>(x), endpoint, e,
                                                                        width, static_cast<uint16_t*>(out));
    }
    return launch_status();
}

extern "C" int gga_edge_values_bwd(int32_t n, int32_t width, int64_t e, const int32_t* row_ptr, const int32_t* eid,
                                   const float* d_edge, float* dx, void* stream) {
    if (n < 0 || width < 1 || e < 0) return GGA_EINVAL;
    if (e >= (int64_t)INT32_MAX) return GGA_ERANGE;
    if (n == 0) return GGA_OK;
    if (!row_ptr || !dx || (e > 0 && (!eid || !d_edge))) return GGA_EINVAL;
    int lw = 1;
    while (lw < width && lw < 64) lw <<= 1;
    int lw_log2 = 0;
    while ((1 << lw_log2) < lw) lw_log2++;
    hipStream_t s = as_stream(stream);
    edge_scatter_sum<<<(unsigned)(((int64_t)n + 3) / 4), 256, 0, s>>>(n, width, lw_log2, row_ptr, eid, d_edge, dx);
    return launch_status();
}

extern "C" int gga_gat_coef_fwd(int32_t n, int32_t heads, int32_t head_dim, const float* hf, const float* a_s,
                                const float* a_t, float* s_src, float* s_dst, void* stream) {
    if (n < 0 || heads < 1 || head_dim < 1) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!hf || !a_s || !s_src || (a_t != nullptr) != (s_dst != nullptr)) return GGA_EINVAL;
    const int64_t nh = (int64_t)n * heads;
    const int vec = head_dim % 4 == 0 && aligned16(hf);
    coef_fwd<<<grid_for(nh, 256), 256, 0, as_stream(stream)>>>(nh, heads, head_dim, hf, a_s, a_t, s_src, s_dst, vec);
    return launch_status();
}

extern "C" size_t gga_gat_coef_bwd_workspace(int32_t n, int32_t heads, int32_t head_dim) {
    if (n < 0 || heads < 1 || head_dim < 1) return 0;
    return align_up((size_t)coef_blocks(n) * 2 * heads * head_dim * sizeof(float), 256);
}

extern "C" int gga_gat_coef_bwd(int32_t n, int32_t heads, int32_t head_dim, const float* hf, const float* a_s,
                                const float* a_t, const float* d_hf_attn, const float* d_s_src, const float* d_s_dst,
                                float* d_hf, float* d_a_s, float* d_a_t, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || heads < 1 || head_dim < 1) return GGA_EINVAL;
    if (!a_s || !d_a_s) return GGA_EINVAL;
    const bool tgt = a_t != nullptr;  // the target side is all present or all absent
    if (tgt != (d_a_t != nullptr) || (n > 0 && tgt != (d_s_dst != nullptr))) return GGA_EINVAL;
    if (n > 0 && (!hf || !d_s_src || !d_hf)) return GGA_EINVAL;
    const size_t need = gga_gat_coef_bwd_workspace(n, heads, head_dim);
    if (ws_bytes < need || !ws) return GGA_EWORKSPACE;
    hipStream_t s = as_stream(stream);
    const int W = heads * head_dim;
    float* part = static_cast<float*>(ws);
    const int nb = coef_blocks(n);
    coef_bwd_partial<<<nb, 256, 0, s>>>(n, heads, head_dim, hf, a_s, a_t, d_hf_attn, d_s_src, d_s_dst, d_hf,
                                                 part);
    coef_bwd_reduce<<<(unsigned)(2 * W), 256, 0, s>>>(W, nb, part, d_a_s, d_a_t);
    return launch_status();
}

extern "C" int gga_head_mean(int32_t n, int32_t heads, int32_t head_dim, const float* in, float* out, void* stream) {
    if (n < 0 || heads < 1 || head_dim < 1) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!in || !out) return GGA_EINVAL;
    const int64_t nc = (int64_t)n * head_dim;
    head_mean_kernel<<<grid_for(nc, 256), 256, 0, as_stream(stream)>>>(nc, heads, head_dim, in, out);
    return launch_status();
}

extern "C" int gga_head_mean_bwd(int32_t n, int32_t heads, int32_t head_dim, const float* d_out, float* d_in,
                                 void* stream) {
    if (n < 0 || heads < 1 || head_dim < 1) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!d_out || !d_in) return GGA_EINVAL;
    const int64_t total = (int64_t)n * heads * head_dim;
    head_mean_bwd_kernel<<<grid_for(total, 256), 256, 0, as_stream(stream)>>>(total, heads, head_dim, d_out, d_in);
    return launch_status();
}
