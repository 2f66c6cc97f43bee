// Fused local attention forward: per target row, gather source rows, score, online
// softmax and weighted aggregation in one pass ("Gated Local-Global Graph Attention",
// Key formulas, local branch; Tinymesh "Sparse attention experiment", sections
// "Target softmax" and "Multiple heads are composition").
//
// Lane layout.  A row of W = H*C elements is covered by LPR lanes holding EPL elements
// each (16-byte loads on the fast path), HDP lanes per head (padded to a power of two),
// and NS slots per lane when one wavefront is not wide enough.  The 64/LPR groups of a
// wavefront take different edges of the same row; their states are merged at the end.
// Scores are kept in log2 units (the score multiplier includes log2(e)), so the
// softmax uses exp2.  No floating-point atomics: every sum has a fixed order.
#include <atomic>
#include <mutex>

#include "plan.hpp"
#include "rowgeo.hpp"
#include "shape.hpp"

namespace gga {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = 64 * kFwdWaves;

struct FwdParams {
    const void* qs;
    const void* ks;
    const void* v;
    const int32_t* row_ptr;
    const int32_t* col;
    const PlanHeader* hdr;
    const int4* light;
    const int4* chunks;
    const int4* heavy;
    float* out;
    float* lse;
    float* part;
    int32_t n, H, C, W;
    int32_t e;  // edges the plan must have been built for
    int32_t lpr_log2;
    int32_t part_stride;
    float score_mul;
    float slope;
    int32_t chunk_blocks;
    int32_t own_rows;    // light rows: each edge group of a wavefront takes a row of its own
    const float* se;     // kScoreAddEdge: edge term of the logit, COO order [E, H]
    const int32_t* eid;  // kScoreAddEdge: COO index of each CSR position
};

// UMAX: edge slots per lane and iteration over the NS row slots.  A row that fills the
// wavefront keeps 8 edges in flight per lane; a row narrower than the wavefront (several
// edge groups per wavefront) keeps 4, which leaves registers for more resident wavefronts.
template <typename T, int EPL, int HDP, int NS, int MODE, int UMAX>
struct FwdRow {
    using V = Vec<T, EPL>;
    using raw_t = typename V::raw_t;
    static constexpr int kUMax = UMAX / NS;

    RowGeo<EPL, HDP, NS> geo;
    int lane, g, G, U, EIT, lpr;
    int off[NS], head[NS];
    bool ok[NS], lead[NS];
    // state
    float m[NS], l[NS], acc[NS][EPL];
    // destination-side operand
    float qf[NS][EPL];
    float sd[NS];

    __device__ __forceinline__ void geometry(const FwdParams& p) {
        geo.init(p.lpr_log2, p.H, p.C);
        lane = geo.lane;
        lpr = geo.lpr;
        G = geo.G;
        g = geo.g;
        U = G * kUMax <= 64 ? kUMax : 64 / G;  // edges per group per iteration: all slots, at most 64 per wave
        EIT = G * U;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            off[s] = geo.off[s];
            head[s] = geo.head[s];
            ok[s] = geo.ok[s];
            lead[s] = geo.lead[s];
        }
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            m[s] = kNegInf;
            l[s] = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; i++) acc[s][i] = 0.f;
        }
    }

    __device__ __forceinline__ void load_target(const FwdParams& p, int32_t v) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if constexpr (MODE == GGA_SCORE_DOT) {
                raw_t r{};
                if (ok[s]) r = load_once(reinterpret_cast<const raw_t*>(static_cast<const T*>(p.qs) + (size_t)v * p.W + off[s]));
                V::widen(r, qf[s]);
            } else if constexpr (MODE != GGA_SCORE_MEAN) {
                sd[s] = ok[s] ? static_cast<const float*>(p.qs)[(size_t)v * p.H + head[s]] : 0.f;
            }
        }
    }

    // Shared row (OWN false): the groups take the edges at positions
    // beg + start + k*stride + (g + G*j), j < U, for k = 0, 1, ... while inside [beg, end).
    // Own rows (OWN true): group g alone takes the edges of its own row [beg, end) (beg and
    // end differ by group), beg + k*U + j, for k < iters (the same for the wavefront).
    template <bool OWN>
    __device__ __forceinline__ void run_t(const FwdParams& p, int32_t beg, int32_t end, int32_t start,
                                          int32_t stride, int32_t iters) {
        const T* __restrict__ kp = static_cast<const T*>(p.ks);
        const T* __restrict__ vp = static_cast<const T*>(p.v);
        const float* __restrict__ ssrc = static_cast<const float*>(p.ks);
        // lane `ll` loads the id of the iteration's edge `ll` (of the wavefront, or of its group)
        const int ll = OWN ? (lane & (lpr - 1)) : lane;
        const int lim = OWN ? U : EIT;
        const int g0 = OWN ? g * lpr : 0;
        int32_t base = beg + start;
        int32_t colv = (ll < lim && base + ll < end) ? p.col[base + ll] : 0;
        int32_t eidv = 0;  // edge terms: the COO index of each position, loaded like col
        if constexpr (MODE == kScoreAddEdge) eidv = (ll < lim && base + ll < end) ? p.eid[base + ll] : 0;
        for (int32_t k = 0; OWN ? k < iters : base < end; k++, base += stride) {
            // the next iteration's sources, in flight while this iteration's rows are gathered
            const int32_t nxt = base + stride;
            const int32_t coln = (ll < lim && nxt + ll < end) ? p.col[nxt + ll] : 0;
            int32_t eidn = 0;
            if constexpr (MODE == kScoreAddEdge) eidn = (ll < lim && nxt + ll < end) ? p.eid[nxt + ll] : 0;
            int32_t u[kUMax], ej[kUMax];
            bool ev[kUMax];
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
                if (j < U) {
                    const int idx = OWN ? g0 + j : g + G * j;
                    u[j] = __shfl(colv, idx, 64);
                    ej[j] = MODE == kScoreAddEdge ? __shfl(eidv, idx, 64) : 0;
                    ev[j] = base + (OWN ? j : idx) < end;
                } else {
                    u[j] = 0;
                    ej[j] = 0;
                    ev[j] = false;
                }
            }
            raw_t kr[kUMax][NS], vr[kUMax][NS];
            float ss[kUMax][NS];
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    kr[j][s] = raw_t{};
                    vr[j][s] = raw_t{};
                    ss[j][s] = 0.f;
                    if (ev[j] && ok[s]) {
                        const size_t ro = (size_t)u[j] * p.W + off[s];
                        if constexpr (MODE == GGA_SCORE_DOT) {
                            kr[j][s] = *reinterpret_cast<const raw_t*>(kp + ro);
                        } else if constexpr (MODE != GGA_SCORE_MEAN) {
                            ss[j][s] = ssrc[(size_t)u[j] * p.H + head[s]];
                            if constexpr (MODE == kScoreAddEdge) ss[j][s] += p.se[(size_t)ej[j] * p.H + head[s]];
                        }
                        vr[j][s] = *reinterpret_cast<const raw_t*>(vp + ro);
                    }
                }
            }
            float sc[kUMax][NS];
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    if (j < U) {
                        float t;
                        if constexpr (MODE == GGA_SCORE_MEAN) {
                            t = 0.f;
                        } else if constexpr (MODE == GGA_SCORE_DOT) {
                            float f[EPL];
                            V::widen(kr[j][s], f);
                            float d = 0.f;
#pragma unroll
                            for (int i = 0; i < EPL; i++) d = fmaf(qf[s][i], f[i], d);
                            t = group_sum<HDP>(d) * p.score_mul;
                        } else {
                            float z = ss[j][s] + sd[s];
                            z = z > 0.f ? z : z * p.slope;
                            t = z * p.score_mul;
                        }
                        sc[j][s] = ev[j] ? t : kNegInf;
                    } else {
                        sc[j][s] = kNegInf;
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < NS; s++) {
                float mx = kNegInf;
#pragma unroll
                for (int j = 0; j < kUMax; j++) mx = fmaxf(mx, sc[j][s]);
                const float mn = fmaxf(m[s], mx);
                if (mn > kNegInf) {
                    const float corr = fexp2(m[s] - mn);
                    l[s] *= corr;
#pragma unroll
                    for (int i = 0; i < EPL; i++) acc[s][i] *= corr;
#pragma unroll
                    for (int j = 0; j < kUMax; j++) {
                        if (j < U) {
                            const float pj = fexp2(sc[j][s] - mn);
                            float f[EPL];
                            V::widen(vr[j][s], f);
                            l[s] += pj;
#pragma unroll
                            for (int i = 0; i < EPL; i++) acc[s][i] = fmaf(pj, f[i], acc[s][i]);
                        }
                    }
                    m[s] = mn;
                }
            }
            colv = coln;
            if constexpr (MODE == kScoreAddEdge) eidv = eidn;
        }
    }

    __device__ __forceinline__ void run(const FwdParams& p, int32_t beg, int32_t end, int32_t start,
                                        int32_t stride) {
        run_t<false>(p, beg, end, start, stride, 0);
    }

    __device__ __forceinline__ void fold(float mo, float lo, const float* ao, int s) {
        const float mn = fmaxf(m[s], mo);
        if (mn > kNegInf) {
            const float a = fexp2(m[s] - mn), b = fexp2(mo - mn);
            l[s] = l[s] * a + lo * b;
#pragma unroll
            for (int i = 0; i < EPL; i++) acc[s][i] = acc[s][i] * a + ao[i] * b;
            m[s] = mn;
        }
    }

    // Butterfly over the G groups of the wavefront; group 0 ends with the whole state.
    __device__ __forceinline__ void merge_groups() {
        for (int o = lpr; o < 64; o <<= 1) {
#pragma unroll
            for (int s = 0; s < NS; s++) {
                const float mo = __shfl_xor(m[s], o, 64);
                const float lo = __shfl_xor(l[s], o, 64);
                float ao[EPL];
#pragma unroll
                for (int i = 0; i < EPL; i++) ao[i] = __shfl_xor(acc[s][i], o, 64);
                fold(mo, lo, ao, s);
            }
        }
    }

    __device__ __forceinline__ void write_final(const FwdParams& p, int32_t v) {
        if (geo.exact) {
            // every lane takes part in the row store (it exchanges chunks across lanes)
            const float inv = l[0] > 0.f ? 1.0f / l[0] : 0.f;
            float o[EPL];
#pragma unroll
            for (int i = 0; i < EPL; i++) o[i] = acc[0][i] * inv;
            store_row_nt<EPL>(p.out + (size_t)v * p.W, o, lpr, lane, g);
            if (g == 0 && lead[0] && p.lse)
                p.lse[(size_t)v * p.H + head[0]] = l[0] > 0.f ? (m[0] + __log2f(l[0])) * kLn2 : kNegInf;
            return;
        }
        if (g != 0) return;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (!ok[s]) continue;
            const float inv = l[s] > 0.f ? 1.0f / l[s] : 0.f;
            float o[EPL];
#pragma unroll
            for (int i = 0; i < EPL; i++) o[i] = acc[s][i] * inv;
            store_f32<EPL>(p.out + (size_t)v * p.W + off[s], o);
            if (lead[s] && p.lse)
                p.lse[(size_t)v * p.H + head[s]] = l[s] > 0.f ? (m[s] + __log2f(l[s])) * kLn2 : kNegInf;
        }
    }

    // Own rows: every group writes its own row v (one slot); `valid` false for a group
    // without a row.  All 64 lanes must call it (the exact layout exchanges values
    // within each group so that a store covers consecutive 16-byte chunks of a row).
    __device__ __forceinline__ void write_own(const FwdParams& p, int32_t v, bool valid) {
        const float inv = l[0] > 0.f ? 1.0f / l[0] : 0.f;
        float o[EPL];
#pragma unroll
        for (int i = 0; i < EPL; i++) o[i] = acc[0][i] * inv;
        float* row = p.out + (size_t)v * p.W;
        if (geo.exact) {
            store_group_row_nt<EPL>(row, o, lpr, lane, valid);
        } else if (valid && ok[0]) {
            store_f32<EPL>(row + off[0], o);
        }
        if (valid && lead[0] && ok[0] && p.lse)
            p.lse[(size_t)v * p.H + head[0]] = l[0] > 0.f ? (m[0] + __log2f(l[0])) * kLn2 : kNegInf;
    }

    __device__ __forceinline__ void write_partial(const FwdParams& p, int32_t slot) {
        if (g != 0) return;
        float* sp = p.part + (size_t)slot * p.part_stride;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (!ok[s]) continue;
            store_f32<EPL>(sp + off[s], acc[s]);
            if (lead[s]) {
                sp[p.W + head[s]] = m[s];
                sp[p.W + p.H + head[s]] = l[s];
            }
        }
    }
};

template <typename T, int EPL, int HDP, int NS, int MODE, int UMAX>
__global__ __launch_bounds__(kFwdThreads) void local_fwd_kernel(FwdParams p) {
    using Row = FwdRow<T, EPL, HDP, NS, MODE, UMAX>;
    if (!plan_usable(p.hdr, p.n, p.e)) return;
    Row r;
    r.geometry(p);
    const int wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < p.chunk_blocks) {
        // one workgroup per chunk of a long row; the four wavefronts interleave the
        // chunk's edges and their states are folded in wavefront order
        __shared__ float sm[kFwdWaves][NS][64][EPL + 2];
        const int nch = p.hdr->n_chunks;
        for (int c = blockIdx.x; c < nch; c += p.chunk_blocks) {
            const int4 ch = p.chunks[c];
            r.reset();
            r.load_target(p, ch.x);
            r.run(p, ch.y, ch.z, wave * r.EIT, kFwdWaves * r.EIT);
            r.merge_groups();
            if (wave > 0) {
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    sm[wave][s][r.lane][0] = r.m[s];
                    sm[wave][s][r.lane][1] = r.l[s];
#pragma unroll
                    for (int i = 0; i < EPL; i++) sm[wave][s][r.lane][2 + i] = r.acc[s][i];
                }
            }
            __syncthreads();
            if (wave == 0) {
                for (int w = 1; w < kFwdWaves; w++) {
#pragma unroll
                    for (int s = 0; s < NS; s++) {
                        float ao[EPL];
#pragma unroll
                        for (int i = 0; i < EPL; i++) ao[i] = sm[w][s][r.lane][2 + i];
                        r.fold(sm[w][s][r.lane][0], sm[w][s][r.lane][1], ao, s);
                    }
                }
                if (ch.w < 0)
                    r.write_final(p, ch.x);
                else
                    r.write_partial(p, ch.w);
            }
            __syncthreads();
        }
        return;
    }
    const int nl = p.hdr->n_light;
    // (light rows narrower than a wavefront: one slot, four edge slots per lane)
    if (NS == 1 && UMAX == 4 && p.own_rows) {
        // the wavefront owns G consecutive light rows
        const int li0 = ((blockIdx.x - p.chunk_blocks) * kFwdWaves + wave) * r.G;
        if (li0 >= nl) return;
        if ((int64_t)p.hdr->light_sum > (int64_t)nl * r.EIT) {
            // light rows longer than one iteration on average: one after another, every
            // group on each
            const int lend = min(li0 + r.G, nl);
            for (int li = li0; li < lend; li++) {
                const int4 lr = p.light[li];
                r.reset();
                r.load_target(p, lr.x);
                r.run(p, lr.y, lr.z, 0, r.EIT);
                r.merge_groups();
                r.write_final(p, lr.x);
            }
            return;
        }
        // short rows: each group takes one of them
        const int li = li0 + r.g;
        const bool valid = li < nl;
        const int4 lr = valid ? p.light[li] : make_int4(0, 0, 0, 0);
        int32_t iters = (lr.z - lr.y + r.U - 1) / r.U;
        for (int o = r.lpr; o < 64; o <<= 1) iters = max(iters, __shfl_xor(iters, o, 64));
        r.reset();
        r.load_target(p, lr.x);
        r.template run_t<true>(p, lr.y, lr.z, 0, r.U, iters);
        r.write_own(p, lr.x, valid);
        return;
    }
    const int li = (blockIdx.x - p.chunk_blocks) * kFwdWaves + wave;
    if (li >= nl) return;
    const int4 lr = p.light[li];
    const int32_t v = lr.x;
    r.reset();
    r.load_target(p, v);
    r.run(p, lr.y, lr.z, 0, r.EIT);
    r.merge_groups();
    r.write_final(p, v);
}

// Folds the partial states of each heavy row in slot order.  A lane holds kMergeCols
// columns (lane + 64 c) of the row at once, and the loads of kMergeBatch slots are issued
// before their folds, so a row of S slots takes about S / kMergeBatch memory round trips
// per 64 * kMergeCols columns.
constexpr int kMergeBatch = 8, kMergeCols = 4;

__global__ __launch_bounds__(kFwdThreads) void local_fwd_merge(FwdParams p) {
    if (!plan_usable(p.hdr, p.n, p.e)) return;
    const int lane = threadIdx.x & 63;
    const int nh = p.hdr->n_heavy;
    for (int hr = blockIdx.x * kFwdWaves + (threadIdx.x >> 6); hr < nh; hr += gridDim.x * kFwdWaves) {
        const int4 hv = p.heavy[hr];
        for (int x0 = 0; x0 < p.W; x0 += 64 * kMergeCols) {
            int h[kMergeCols];
            bool in[kMergeCols];
            float m[kMergeCols], l[kMergeCols], a[kMergeCols];
#pragma unroll
            for (int c = 0; c < kMergeCols; c++) {
                const int x = x0 + lane + 64 * c;
                in[c] = x < p.W;
                h[c] = in[c] ? x / p.C : 0;
                m[c] = kNegInf;
                l[c] = a[c] = 0.f;
            }
            for (int i0 = 0; i0 < hv.z; i0 += kMergeBatch) {
                float mi[kMergeBatch][kMergeCols], li[kMergeBatch][kMergeCols], ai[kMergeBatch][kMergeCols];
#pragma unroll
                for (int j = 0; j < kMergeBatch; j++) {
                    const float* sp = p.part + (size_t)(hv.y + i0 + j) * p.part_stride;
#pragma unroll
                    for (int c = 0; c < kMergeCols; c++) {
                        mi[j][c] = kNegInf;
                        li[j][c] = ai[j][c] = 0.f;
                        if (i0 + j < hv.z && in[c]) {
                            mi[j][c] = sp[p.W + h[c]];
                            li[j][c] = sp[p.W + p.H + h[c]];
                            ai[j][c] = sp[x0 + lane + 64 * c];
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < kMergeBatch; j++) {
                    if (i0 + j >= hv.z) break;
#pragma unroll
                    for (int c = 0; c < kMergeCols; c++) {
                        const float mn = fmaxf(m[c], mi[j][c]);
                        if (mn > kNegInf) {
                            const float ca = fexp2(m[c] - mn), cb = fexp2(mi[j][c] - mn);
                            l[c] = l[c] * ca + li[j][c] * cb;
                            a[c] = a[c] * ca + ai[j][c] * cb;
                            m[c] = mn;
                        }
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < kMergeCols; c++) {
                if (!in[c]) continue;
                const int x = x0 + lane + 64 * c;
                p.out[(size_t)hv.x * p.W + x] = l[c] > 0.f ? a[c] * (1.0f / l[c]) : 0.f;
                if (p.lse && x - h[c] * p.C == 0)
                    p.lse[(size_t)hv.x * p.H + h[c]] = l[c] > 0.f ? (m[c] + __log2f(l[c])) * kLn2 : kNegInf;
            }
        }
    }
}

// ---------------------------------------------------------------- host side

size_t part_stride(int H, int C) { return align_up((size_t)H * C + 2 * (size_t)H, 8); }

template <typename T, int EPL, int HDP, int NS, int MODE, int UMAX>
void launch(const FwdParams& p, unsigned grid, int64_t max_heavy, hipStream_t s) {
    local_fwd_kernel<T, EPL, HDP, NS, MODE, UMAX><<<grid, kFwdThreads, 0, s>>>(p);
    if (max_heavy > 0) {
        int64_t mb = (max_heavy + kFwdWaves - 1) / kFwdWaves;
        unsigned mg = (unsigned)(mb < 1024 ? mb : 1024);
        local_fwd_merge<<<mg, kFwdThreads, 0, s>>>(p);
    }
}

template <typename T, int EPL, int MODE>
bool dispatch_hdp(const Shape& sh, const FwdParams& p, unsigned grid, int64_t mh, hipStream_t s) {
#define GGA_CASE(HD)                                                              \
    case HD:                                                                      \
        if (sh.ns == 1 && sh.lpr_log2 == 6)                                       \
            launch<T, EPL, HD, 1, MODE, 8>(p, grid, mh, s);                       \
        else if (sh.ns == 1)                                                      \
            launch<T, EPL, HD, 1, MODE, 4>(p, grid, mh, s);                       \
        else if constexpr (EPL > 1)                                               \
            launch<T, EPL, HD, 2, MODE, 8>(p, grid, mh, s);                       \
        else                                                                      \
            return false;                                                         \
        return true;
    switch (sh.hdp) {
        GGA_CASE(1)
        GGA_CASE(2)
        GGA_CASE(4)
        GGA_CASE(8)
        GGA_CASE(16)
        GGA_CASE(32)
        GGA_CASE(64)
        default:
            return false;
    }
#undef GGA_CASE
}

template <int MODE>
bool dispatch(int dtype, const Shape& sh, const FwdParams& p, unsigned grid, int64_t mh, hipStream_t s) {
    if (dtype == GGA_BF16) {
        if (sh.epl == 8) return dispatch_hdp<uint16_t, 8, MODE>(sh, p, grid, mh, s);
        return dispatch_hdp<uint16_t, 1, MODE>(sh, p, grid, mh, s);
    }
    if (sh.epl == 4) return dispatch_hdp<float, 4, MODE>(sh, p, grid, mh, s);
    return dispatch_hdp<float, 1, MODE>(sh, p, grid, mh, s);
}

// The additive score with an edge term: fp32 node tensors only.
bool dispatch_edge(int dtype, const Shape& sh, const FwdParams& p, unsigned grid, int64_t mh, hipStream_t s) {
    if (dtype != GGA_F32) return false;
    if (sh.epl == 4) return dispatch_hdp<float, 4, kScoreAddEdge>(sh, p, grid, mh, s);
    return dispatch_hdp<float, 1, kScoreAddEdge>(sh, p, grid, mh, s);
}

size_t fwd_part_bytes(const gga_local_desc* d) {
    PlanBounds b = plan_bounds(d->e);
    return align_up((size_t)b.max_slots * part_stride(d->heads, d->head_dim) * sizeof(float), 256);
}

// The forward with an optional edge term `se` (CSR order); ws holds the split-row partials.
int fwd_impl(const gga_local_desc* d, const void* qs, const void* ks, const void* v, const int32_t* row_ptr,
             const int32_t* col, const void* plan, float* out, float* lse, const float* se, const int32_t* eid, void* ws,
             size_t ws_bytes, hipStream_t s) {
    const bool mean = d->score == GGA_SCORE_MEAN;
    if (!row_ptr || !plan || !out || (!qs && !mean)) return GGA_EINVAL;
    if (d->e > 0 && (!col || (!ks && !mean) || !v)) return GGA_EINVAL;
    if (!aligned16(out) || !aligned16(qs) || (ks && !aligned16(ks)) || (v && !aligned16(v))) return GGA_EINVAL;
    const size_t need = fwd_part_bytes(d);
    if (ws_bytes < need || (need > 0 && !ws)) return GGA_EWORKSPACE;
    Shape sh;
    pick_shape(d->heads, d->head_dim, d->dtype, &sh);

    PlanView pv = plan_view(const_cast<void*>(plan), d->n, d->e);
    PlanBounds b = plan_bounds(d->e);
    FwdParams p{};
    p.qs = qs;
    p.ks = ks;
    p.v = v;
    p.row_ptr = row_ptr;
    p.col = col;
    p.hdr = pv.hdr;
    p.light = pv.light;
    p.chunks = pv.chunks;
    p.heavy = pv.heavy;
    p.out = out;
    p.lse = lse;
    p.part = static_cast<float*>(ws);
    p.se = se;
    p.eid = eid;
    p.n = d->n;
    p.e = (int32_t)d->e;
    p.H = d->heads;
    p.C = d->head_dim;
    p.W = d->heads * d->head_dim;
    p.lpr_log2 = sh.lpr_log2;
    p.part_stride = (int32_t)part_stride(d->heads, d->head_dim);
    const float log2e = 1.44269504088896340736f;
    p.score_mul = d->score == GGA_SCORE_DOT ? d->scale * log2e : log2e;
    p.slope = d->negative_slope;
    const int64_t cb = b.max_chunks < 2048 ? b.max_chunks : 2048;
    p.chunk_blocks = d->e > kLightEdges ? (int32_t)cb : 0;
    // rows narrower than a wavefront: its edge groups take light rows of their own
    p.own_rows = sh.ns == 1 && sh.lpr_log2 < 6;
    const int64_t rows_per_block = (int64_t)kFwdWaves << (p.own_rows ? 6 - sh.lpr_log2 : 0);
    const int64_t light_blocks = ((int64_t)d->n + rows_per_block - 1) / rows_per_block;
    const int64_t grid = p.chunk_blocks + light_blocks;
    if (grid >= ((int64_t)1 << 31)) return GGA_ERANGE;
    const int64_t mh = d->e > kChunkEdges ? b.max_heavy : 0;
    bool ok;
    if (se)
        ok = dispatch_edge(d->dtype, sh, p, (unsigned)grid, mh, s);
    else if (d->score == GGA_SCORE_DOT)
        ok = dispatch<GGA_SCORE_DOT>(d->dtype, sh, p, (unsigned)grid, mh, s);
    else if (mean)
        ok = dispatch<GGA_SCORE_MEAN>(d->dtype, sh, p, (unsigned)grid, mh, s);
    else
        ok = dispatch<GGA_SCORE_ADDITIVE>(d->dtype, sh, p, (unsigned)grid, mh, s);
    if (!ok) return GGA_EUNSUPPORTED;
    return launch_status();
}

}  // namespace

}  // namespace gga

using namespace gga;

extern "C" size_t gga_local_attn_fwd_workspace(const gga_local_desc* d) {
    if (check_desc(d) != GGA_OK) return 0;
    return fwd_part_bytes(d);
}

extern "C" int gga_local_attn_fwd(const gga_local_desc* d, const void* qs, const void* ks, const void* v,
                                  const int32_t* row_ptr, const int32_t* col, const void* plan, float* out,
                                  float* lse, void* ws, size_t ws_bytes, void* stream) {
    int st = check_desc(d);
    if (st != GGA_OK) return st;
    if (d->n == 0) return GGA_OK;
    return fwd_impl(d, qs, ks, v, row_ptr, col, plan, out, lse, nullptr, nullptr, ws, ws_bytes, as_stream(stream));
}

// ---------------------------------------------------------------- allocation-free forward
//
// gga_local_attn_fwd_noalloc keeps the split-row partial states in `scratch`, a fixed
// array of device memory that each device holds for the life of the process, instead of
// a caller workspace.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the first call on a device looks up that device's
// address of the array once, with the device current, and every later call on the device
// uses the address it keeps.

namespace gga {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(96) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on that device.
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GGA_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GGA_EUNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GGA_EHIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return GGA_OK;
}

}  // namespace
}  // namespace gga

extern "C" int gga_local_attn_fwd_noalloc(const gga_local_desc* d, const void* qs, const void* ks, const void* v,
                                          const int32_t* row_ptr, const int32_t* col, const void* plan, float* out,
                                          float* lse, void* stream) {
    int st = check_desc(d);
    if (st != GGA_OK) return st;
    // the partial states of every row split into chunks must fit the fixed array
    const size_t need = fwd_part_bytes(d);
    if (need > kNoAllocScratchBytes) return GGA_ESCRATCH;
    if (d->n == 0) return GGA_OK;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != GGA_OK) return st;
    return fwd_impl(d, qs, ks, v, row_ptr, col, plan, out, lse, nullptr, nullptr, ws, kNoAllocScratchBytes,
                    as_stream(stream));
}

extern "C" size_t gga_local_attn_fwd_edge_workspace(const gga_local_desc* d) {
    if (check_desc(d) != GGA_OK) return 0;
    return fwd_part_bytes(d);
}

extern "C" int gga_local_attn_fwd_edge(const gga_local_desc* d, const float* s_dst, const float* s_src,
                                       const void* hf, const float* s_edge, const int32_t* row_ptr,
                                       const int32_t* col, const int32_t* eid, const void* plan, float* out,
                                       float* lse, void* ws, size_t ws_bytes, void* stream) {
    int st = check_desc(d);
    if (st != GGA_OK) return st;
    if (d->score != GGA_SCORE_ADDITIVE || d->dtype != GGA_F32) return GGA_EUNSUPPORTED;
    if (d->n == 0) return GGA_OK;
    if (d->e > 0 && (!s_edge || !eid)) return GGA_EINVAL;
    // the kernel reads each edge's term in COO order through eid
    return fwd_impl(d, s_dst, s_src, hf, row_ptr, col, plan, out, lse, d->e > 0 ? s_edge : nullptr, eid, ws,
                    ws_bytes, as_stream(stream));
}
