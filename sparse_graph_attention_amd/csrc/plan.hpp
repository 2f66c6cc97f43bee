// Layout of the degree-bucket plan (an opaque device buffer to callers).
#pragma once

#include "common.hpp"

namespace gga {

// Rows with at most kLightEdges in-edges are processed by one wavefront each.  Longer
// rows are cut into chunks of at most kChunkEdges edges, one workgroup per chunk; when
// a row has more than one chunk, each chunk leaves a partial softmax state in a slot and
// a merge kernel folds the row's slots in slot order.
constexpr int kLightEdges = 64;
constexpr int kChunkEdges = 1024;

struct PlanHeader {
    int32_t n_light;   // rows in the light list
    int32_t n_chunks;  // entries of the chunk table
    int32_t n_heavy;   // rows cut into more than one chunk
    int32_t n_slots;   // partial-state slots used by those rows
    int32_t n;         // rows the plan was built for
    int32_t light_edges;
    int32_t chunk_edges;
    int32_t magic;
    int32_t light_sum;  // edges of the light rows together (their mean length picks a lane layout)
    int32_t e;          // edges the plan was built for
    int32_t status;     // 0, or GGA_ERANGE when a row of row_ptr lies outside [0, e] or the rows overflow e
    int32_t misuse;     // set by a kernel handed this plan with other sizes than it was built for
};

constexpr int32_t kPlanMagic = 0x67676150;

struct PlanBounds {
    int64_t max_chunks, max_heavy, max_slots;
};

inline PlanBounds plan_bounds(int64_t e) {
    PlanBounds b;
    b.max_chunks = e / (kLightEdges + 1) + e / kChunkEdges + 1;
    b.max_heavy = e / (kChunkEdges + 1) + 1;
    b.max_slots = e / kChunkEdges + e / (kChunkEdges + 1) + 1;
    return b;
}

// Device views into a plan buffer.
struct PlanView {
    PlanHeader* hdr;
    int4* light;     // [n]: row, begin, end, 0 (the row's edge range read with its id)
    int4* chunks;    // [max_chunks]: row, begin, end, slot (-1: chunk is the whole row)
    int4* heavy;     // [max_heavy]: row, first slot, slot count, 0
    size_t bytes;
};

// A kernel over `rows` rows and `edges` edges uses a plan only when it is a plan, built for
// those sizes, from a row_ptr whose rows lie within [0, edges].  Any other plan reads as
// empty: the kernel processes no row and writes nothing, so no table or column index is
// read out of bounds; the first thread of the grid records the misuse in the plan.
__device__ __forceinline__ bool plan_usable(const PlanHeader* h, int32_t rows, int64_t edges) {
    const bool ok = h->magic == kPlanMagic && h->status == 0 && h->n == rows && (int64_t)h->e == edges;
    if (!ok && blockIdx.x == 0 && threadIdx.x == 0 && h->magic == kPlanMagic)
        const_cast<PlanHeader*>(h)->misuse = 1;
    return ok;
}

inline PlanView plan_view(void* plan, int32_t n, int64_t e) {
    PlanBounds b = plan_bounds(e);
    Carver c(plan);
    PlanView v;
    v.hdr = c.take<PlanHeader>(1);
    v.light = c.take<int4>((size_t)n);
    v.chunks = c.take<int4>((size_t)b.max_chunks);
    v.heavy = c.take<int4>((size_t)b.max_heavy);
    v.bytes = c.bytes();
    return v;
}

}  // namespace gga
