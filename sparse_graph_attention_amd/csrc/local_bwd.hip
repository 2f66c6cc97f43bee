// Host entry point of the local attention backward (kernels in local_bwd_impl.hpp).
#include "local_bwd_impl.hpp"
#include "shape.hpp"

namespace gga {
namespace {

struct BwdWs {
    float* D;
    float* part_a;
    float* part_b;
    int32_t stride_a, stride_b;
    size_t bytes;
};

// Width of the score-side gradients: q/k rows (dot), one value per head (additive),
// none (mean).
int64_t score_width(const gga_local_desc* d) {
    const int64_t W = (int64_t)d->heads * d->head_dim;
    return d->score == GGA_SCORE_DOT ? W : d->score == GGA_SCORE_MEAN ? 0 : d->heads;
}

BwdWs carve_bwd(void* ws, const gga_local_desc* d) {
    const PlanBounds b = plan_bounds(d->e);
    const int64_t W = (int64_t)d->heads * d->head_dim;
    const int64_t wk = score_width(d);
    BwdWs w;
    w.stride_a = (int32_t)align_up((size_t)wk, 8);
    w.stride_b = (int32_t)(align_up((size_t)wk, 8) + align_up((size_t)W, 8));
    Carver c(ws);
    w.D = c.take<float>((size_t)d->n * d->heads);
    w.part_a = c.take<float>((size_t)b.max_slots * w.stride_a);
    w.part_b = c.take<float>((size_t)b.max_slots * w.stride_b);
    w.bytes = c.bytes();
    return w;
}

// The per-edge logit term (COO order) and the CSRs' COO indices through which the passes
// read it; pass A writes dz_e for every edge, in COO order, through the same indices.
struct EdgeTerms {
    const float* se;
    float* dz;
    const int32_t* eid_a;
    const int32_t* eid_b;
};

// No targets: every source-side gradient is zero.
int zero_source_grads(const gga_local_desc* d, float* d_ks, float* d_v, hipStream_t s) {
    const int64_t ns = source_rows(d), wk = score_width(d);
    if (ns == 0) return GGA_OK;
    if (!d_v || (wk > 0 && !d_ks)) return GGA_EINVAL;
    if (wk > 0) fill_f32(d_ks, ns * wk, 0.f, s);
    fill_f32(d_v, ns * (int64_t)d->heads * d->head_dim, 0.f, s);
    return launch_status();
}

int bwd_impl(const gga_local_desc* d, const void* qs, const void* ks, const void* v, const float* out,
             const float* lse, const float* d_out, const int32_t* row_ptr, const int32_t* col, const void* plan,
             const int32_t* row_ptr_s, const int32_t* col_s, const void* plan_s, float* d_qs, float* d_ks,
             float* d_v, const EdgeTerms* et, void* ws, size_t ws_bytes, hipStream_t s) {
    const bool mean = d->score == GGA_SCORE_MEAN;
    if (!d_out || !row_ptr || !plan || !row_ptr_s || !plan_s || !d_v) return GGA_EINVAL;
    if (!mean && (!qs || !out || !lse || !d_qs || !d_ks)) return GGA_EINVAL;
    if (d->e > 0 && (!col || !col_s || (!mean && (!ks || !v)))) return GGA_EINVAL;
    for (const void* p : {qs, ks, v, (const void*)out, (const void*)d_out, (const void*)d_qs, (const void*)d_ks,
                          (const void*)d_v})
        if (p && !aligned16(p)) return GGA_EINVAL;
    const BwdWs need = carve_bwd(nullptr, d);
    if (ws_bytes < need.bytes || !ws) return GGA_EWORKSPACE;
    const BwdWs w = carve_bwd(ws, d);
    const int64_t W = (int64_t)d->heads * d->head_dim;
    const int64_t wk = score_width(d);
    const int32_t ns = source_rows(d);
    if (d->e == 0) {
        if (wk > 0) {
            fill_f32(d_qs, (int64_t)d->n * wk, 0.f, s);
            fill_f32(d_ks, (int64_t)ns * wk, 0.f, s);
        }
        fill_f32(d_v, (int64_t)ns * W, 0.f, s);
        return launch_status();
    }
    Shape sh;
    pick_shape(d->heads, d->head_dim, d->dtype, &sh);
    const PlanBounds b = plan_bounds(d->e);
    const PlanView pa = plan_view(const_cast<void*>(plan), d->n, d->e);
    const PlanView pb = plan_view(const_cast<void*>(plan_s), ns, d->e);
    const int64_t cb = b.max_chunks < 2048 ? b.max_chunks : 2048;
    BwdParams p{};
    p.qs = qs;
    p.ks = ks;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.dout = d_out;
    p.d_qs = d_qs;
    p.d_ks = d_ks;
    p.d_v = d_v;
    p.D = w.D;
    p.a = BwdCsr{row_ptr, col, pa.hdr, pa.light, pa.chunks, pa.heavy, w.part_a, w.stride_a,
                 d->e > kLightEdges ? (int32_t)cb : 0, d->n, (int32_t)d->e};
    p.b = BwdCsr{row_ptr_s, col_s, pb.hdr, pb.light, pb.chunks, pb.heavy, w.part_b, w.stride_b,
                 d->e > kLightEdges ? (int32_t)cb : 0, ns, (int32_t)d->e};
    p.n = d->n;
    p.H = d->heads;
    p.C = d->head_dim;
    p.W = (int32_t)W;
    p.lpr_log2 = sh.lpr_log2;
    p.scale = d->scale;
    p.score_mul = d->score == GGA_SCORE_DOT ? d->scale * kLog2e : kLog2e;
    p.slope = d->negative_slope;
    int mode = d->score;
    if (et) {
        p.se = et->se;
        p.dz = et->dz;
        p.eid_a = et->eid_a;
        p.eid_b = et->eid_b;
        mode = kScoreAddEdge;
    }
    // rows narrower than a wavefront: its edge groups take light rows of their own
    p.own_rows = sh.ns == 1 && sh.lpr_log2 < 6;
    const int64_t rows_per_block = (int64_t)kBwdWaves << (p.own_rows ? 6 - sh.lpr_log2 : 0);
    const int64_t light_a = ((int64_t)d->n + rows_per_block - 1) / rows_per_block;
    const int64_t light_b = ((int64_t)ns + rows_per_block - 1) / rows_per_block;
    const int64_t ga = p.a.chunk_blocks + light_a, gb = p.b.chunk_blocks + light_b;
    if (ga >= ((int64_t)1 << 31) || gb >= ((int64_t)1 << 31)) return GGA_ERANGE;
    const int64_t mh = d->e > kChunkEdges ? b.max_heavy : 0;
    const bool ok = d->dtype == GGA_BF16
                        ? launch_bwd_bf16(p, sh.epl, sh.hdp, sh.ns, mode, (unsigned)ga, (unsigned)gb, mh, s)
                        : launch_bwd_f32(p, sh.epl, sh.hdp, sh.ns, mode, (unsigned)ga, (unsigned)gb, mh, s);
    if (!ok) return GGA_EUNSUPPORTED;
    return launch_status();
}

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" size_t gga_local_attn_bwd_workspace(const gga_local_desc* d) {
    if (check_desc(d) != GGA_OK) return 0;
    return carve_bwd(nullptr, d).bytes;
}

extern "C" int gga_local_attn_bwd(const gga_local_desc* d, const void* qs, const void* ks, const void* v,
                                  const float* out, const float* lse, const float* d_out, const int32_t* row_ptr,
                                  const int32_t* col, const void* plan, const int32_t* row_ptr_s,
                                  const int32_t* col_s, const void* plan_s, float* d_qs, float* d_ks, float* d_v,
                                  void* ws, size_t ws_bytes, void* stream) {
    int st = check_desc(d);
    if (st != GGA_OK) return st;
    if (d->n == 0) return zero_source_grads(d, d_ks, d_v, as_stream(stream));
    return bwd_impl(d, qs, ks, v, out, lse, d_out, row_ptr, col, plan, row_ptr_s, col_s, plan_s, d_qs, d_ks, d_v,
                    nullptr, ws, ws_bytes, as_stream(stream));
}

extern "C" size_t gga_local_attn_bwd_edge_workspace(const gga_local_desc* d) {
    if (check_desc(d) != GGA_OK) return 0;
    return carve_bwd(nullptr, d).bytes;
}

extern "C" int gga_local_attn_bwd_edge(const gga_local_desc* d, const float* s_dst, const float* s_src,
                                       const void* hf, const float* s_edge, const float* out, const float* lse,
                                       const float* d_out, const int32_t* row_ptr, const int32_t* col,
                                       const int32_t* eid, const void* plan, const int32_t* row_ptr_s,
                                       const int32_t* col_s, const int32_t* eid_s, const void* plan_s,
                                       float* d_s_dst, float* d_s_src, float* d_hf, float* d_s_edge, void* ws,
                                       size_t ws_bytes, void* stream) {
    int st = check_desc(d);
    if (st != GGA_OK) return st;
    if (d->score != GGA_SCORE_ADDITIVE || d->dtype != GGA_F32) return GGA_EUNSUPPORTED;
    if (d->n == 0) return zero_source_grads(d, d_s_src, d_hf, as_stream(stream));
    if (d->e > 0 && (!s_edge || !eid || !eid_s || !d_s_edge)) return GGA_EINVAL;
    // both passes read the edge term in COO order through the CSRs' eid; pass A writes dz_e
    // straight to d_s_edge in COO order
    const EdgeTerms et{s_edge, d_s_edge, eid, eid_s};
    return bwd_impl(d, s_dst, s_src, hf, out, lse, d_out, row_ptr, col, plan, row_ptr_s, col_s, plan_s, d_s_dst,
                    d_s_src, d_hf, d->e > 0 ? &et : nullptr, ws, ws_bytes, as_stream(stream));
}
