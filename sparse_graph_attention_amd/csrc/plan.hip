// Degree-bucket plan: light rows (one wavefront each), chunked rows (one workgroup per
// chunk) and heavy rows (several chunks merged in a fixed order).  Built from row_ptr
// alone, with device-side counts, so no host read-back is needed.
#include "plan.hpp"

namespace gga {

namespace {

struct PlanWs {
    int32_t* a;  // light flag -> light position
    int32_t* b;  // chunk count -> first chunk
    int32_t* c;  // slot count -> first slot
    int32_t* d;  // heavy flag -> heavy position
    int32_t* e;  // degree of a light row (0 otherwise), summed into the header
    int32_t* scan;
    size_t bytes;
};

PlanWs carve_ws(void* ws, int32_t n) {
    Carver c(ws);
    PlanWs w;
    w.a = c.take<int32_t>((size_t)n);
    w.b = c.take<int32_t>((size_t)n);
    w.c = c.take<int32_t>((size_t)n);
    w.d = c.take<int32_t>((size_t)n);
    w.e = c.take<int32_t>((size_t)n);
    w.scan = c.take<int32_t>(scan_workspace_elems(n));
    w.bytes = c.bytes();
    return w;
}

__global__ void plan_classify(const int32_t* __restrict__ row_ptr, int32_t n, int32_t* a, int32_t* b, int32_t* c,
                              int32_t* d, int32_t* e) {
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < n; v += (int64_t)gridDim.x * blockDim.x) {
        const int32_t deg = row_ptr[v + 1] - row_ptr[v];
        const bool light = deg <= kLightEdges;
        const int32_t chunks = light ? 0 : (deg + kChunkEdges - 1) / kChunkEdges;
        a[v] = light;
        b[v] = chunks;
        c[v] = chunks > 1 ? chunks : 0;
        d[v] = chunks > 1;
        e[v] = light ? deg : 0;
    }
}

__global__ void plan_fill(const int32_t* __restrict__ row_ptr, int32_t n, const int32_t* a, const int32_t* b,
                          const int32_t* c, const int32_t* d, PlanView pv) {
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < n; v += (int64_t)gridDim.x * blockDim.x) {
        const int32_t beg = row_ptr[v], end = row_ptr[v + 1];
        const int32_t deg = end - beg;
        if (deg <= kLightEdges) {
            pv.light[a[v]] = make_int4((int32_t)v, beg, end, 0);
            continue;
        }
        const int32_t chunks = (deg + kChunkEdges - 1) / kChunkEdges;
        const bool heavy = chunks > 1;
        for (int32_t k = 0; k < chunks; k++) {
            const int32_t cb = beg + k * kChunkEdges;
            const int32_t ce = (end - cb) < kChunkEdges ? end : cb + kChunkEdges;
            pv.chunks[b[v] + k] = make_int4((int32_t)v, cb, ce, heavy ? c[v] + k : -1);
        }
        if (heavy) pv.heavy[d[v]] = make_int4((int32_t)v, c[v], chunks, 0);
    }
}

__global__ void plan_header(PlanHeader* hdr, int32_t n) {
    hdr->n = n;
    hdr->light_edges = kLightEdges;
    hdr->chunk_edges = kChunkEdges;
    hdr->magic = kPlanMagic;
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

extern "C" size_t gga_plan_bytes(int32_t n, int64_t e) {
    if (n < 0 || e < 0) return 0;
    return plan_view(nullptr, n, e).bytes;
}

extern "C" size_t gga_plan_workspace(int32_t n, int64_t e) {
    (void)e;
    if (n < 0) return 0;
    return carve_ws(nullptr, n).bytes;
}

extern "C" int gga_plan_build(int32_t n, int64_t e, const int32_t* row_ptr, void* plan, size_t plan_bytes, void* ws,
                              size_t ws_bytes, void* stream) {
    if (n < 0 || e < 0) return GGA_EINVAL;
    if (e >= (int64_t)INT32_MAX) return GGA_ERANGE;
    if (!row_ptr || !plan) return GGA_EINVAL;
    PlanView pv = plan_view(nullptr, n, e);
    if (plan_bytes < pv.bytes) return GGA_EWORKSPACE;
    PlanWs w = carve_ws(nullptr, n);
    if (ws_bytes < w.bytes || (w.bytes > 0 && !ws)) return GGA_EWORKSPACE;
    pv = plan_view(plan, n, e);
    w = carve_ws(ws, n);
    hipStream_t s = as_stream(stream);
    int32_t* hdr_i = reinterpret_cast<int32_t*>(pv.hdr);
    fill_i32(hdr_i, sizeof(PlanHeader) / 4, 0, s);
    plan_header<<<1, 1, 0, s>>>(pv.hdr, n);
    if (n == 0) return launch_status();
    plan_classify<<<grid_for(n), 256, 0, s>>>(row_ptr, n, w.a, w.b, w.c, w.d, w.e);
    exclusive_scan_i32(w.a, w.a, n, &pv.hdr->n_light, w.scan, s);
    exclusive_scan_i32(w.b, w.b, n, &pv.hdr->n_chunks, w.scan, s);
    exclusive_scan_i32(w.c, w.c, n, &pv.hdr->n_slots, w.scan, s);
    exclusive_scan_i32(w.d, w.d, n, &pv.hdr->n_heavy, w.scan, s);
    exclusive_scan_i32(w.e, w.e, n, &pv.hdr->light_sum, w.scan, s);
    plan_fill<<<grid_for(n), 256, 0, s>>>(row_ptr, n, w.a, w.b, w.c, w.d, pv);
    return launch_status();
}
