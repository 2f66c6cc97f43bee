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
        // (64-bit: a row may hold up to 2^31 - 2 edges, and a corrupt row_ptr any difference;
        // plan_fill reports a row with a negative length)
        const int64_t deg = (int64_t)row_ptr[v + 1] - row_ptr[v];
        const bool light = deg <= kLightEdges;
        const int32_t chunks = light ? 0 : (int32_t)((deg + kChunkEdges - 1) / kChunkEdges);
        a[v] = light;
        b[v] = chunks;
        c[v] = chunks > 1 ? chunks : 0;
        d[v] = chunks > 1;
        e[v] = light && deg > 0 ? (int32_t)deg : 0;
    }
}

// Writes each row's entries.  A row outside [0, e], or entries past the tables sized for e
// edges (rows that overlap add up to more than e), are not written: the plan's status
// becomes GGA_ERANGE and every kernel then reads it as empty.
__global__ void plan_fill(const int32_t* __restrict__ row_ptr, int32_t n, int64_t e, PlanBounds bnd, const int32_t* a,
                          const int32_t* b, const int32_t* c, const int32_t* d, PlanView pv) {
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < n; v += (int64_t)gridDim.x * blockDim.x) {
        const int32_t beg = row_ptr[v], end = row_ptr[v + 1];
        if (beg < 0 || end < beg || (int64_t)end > e) {
            pv.hdr->status = GGA_ERANGE;
            continue;
        }
        const int64_t deg = (int64_t)end - beg;
        if (deg <= kLightEdges) {
            pv.light[a[v]] = make_int4((int32_t)v, beg, end, 0);
            continue;
        }
        const int32_t chunks = (int32_t)((deg + kChunkEdges - 1) / kChunkEdges);
        const bool heavy = chunks > 1;
        // the scans' positions are checked at both ends: other rows of a corrupt row_ptr
        // (reported above) may have pushed them out of the tables
        if (b[v] < 0 || (int64_t)b[v] + chunks > bnd.max_chunks ||
            (heavy && (d[v] < 0 || (int64_t)d[v] >= bnd.max_heavy || c[v] < 0 ||
                       (int64_t)c[v] + chunks > bnd.max_slots))) {
            pv.hdr->status = GGA_ERANGE;
            continue;
        }
        for (int32_t k = 0; k < chunks; k++) {
            const int32_t cb = beg + k * kChunkEdges;
            const int32_t ce = (end - cb) < kChunkEdges ? end : cb + kChunkEdges;
            pv.chunks[b[v] + k] = make_int4((int32_t)v, cb, ce, heavy ? c[v] + k : -1);
        }
        if (heavy) pv.heavy[d[v]] = make_int4((int32_t)v, c[v], chunks, 0);
    }
}

// Every field of the header: the sizes, and zero counts and status (the counts come from
// the scans that follow).
__global__ void plan_header(PlanHeader* hdr, int32_t n, int64_t e) {
    PlanHeader h{};
    h.n = n;
    h.e = (int32_t)e;
    h.light_edges = kLightEdges;
    h.chunk_edges = kChunkEdges;
    h.magic = kPlanMagic;
    *hdr = h;
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
    plan_header<<<1, 1, 0, s>>>(pv.hdr, n, e);
    if (n == 0) return launch_status();
    plan_classify<<<grid_for(n), 256, 0, s>>>(row_ptr, n, w.a, w.b, w.c, w.d, w.e);
    ScanCols sc{{w.a, w.b, w.c, w.d, w.e},
                {&pv.hdr->n_light, &pv.hdr->n_chunks, &pv.hdr->n_slots, &pv.hdr->n_heavy, &pv.hdr->light_sum},
                5};
    exclusive_scan_cols(sc, n, w.scan, s);
    plan_fill<<<grid_for(n), 256, 0, s>>>(row_ptr, n, e, plan_bounds(e), w.a, w.b, w.c, w.d, pv);
    return launch_status();
}

namespace gga {
namespace {

__global__ void plan_status_kernel(const PlanHeader* hdr, int32_t n, int64_t e, int32_t* out) {
    int32_t st = GGA_OK;
    if (hdr->magic != kPlanMagic || hdr->n != n || (int64_t)hdr->e != e)
        st = GGA_EINVAL;
    else if (hdr->status != 0)
        st = hdr->status;
    else if (hdr->misuse != 0)
        st = GGA_EINVAL;
    *out = st;
}

}  // namespace
}  // namespace gga

extern "C" int gga_plan_status(const void* plan, int32_t n, int64_t e, int32_t* d_status, void* stream) {
    if (!plan || !d_status || n < 0 || e < 0) return GGA_EINVAL;
    if (e >= (int64_t)INT32_MAX) return GGA_ERANGE;
    plan_status_kernel<<<1, 1, 0, as_stream(stream)>>>(static_cast<const PlanHeader*>(plan), n, e, d_status);
    return launch_status();
}
