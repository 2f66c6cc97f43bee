// Local attention backward, two deterministic passes (no floating-point atomics).
//
// With the softmax maximum held constant (Tinymesh "Sparse attention experiment",
// "Target softmax"), for an edge e: u -> v and head h:
//   alpha_e = exp(s_e - lse[v]),  d alpha_e = dO[v] . v[u],  D[v] = dO[v] . out[v]
//   ds_e = alpha_e (d alpha_e - D[v])
// Pass A walks the CSR by destination: dq[v] (dot) or d s_dst[v] (additive), and D.
// Pass B walks the CSR by source, grouping the edge gradients by their source
// (Tinymesh "Endpoint projection", backward): dk[u] or d s_src[u], and dv[u].
// Mean weighting (alpha_e = 1/deg(v), constant) needs pass B alone, for dv.
// Long rows of either CSR are cut into chunks whose partial sums are added in slot order.
#pragma once

#include <type_traits>

#include "plan.hpp"
#include "rowgeo.hpp"

namespace gga {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;

struct BwdCsr {
    const int32_t* row_ptr;
    const int32_t* col;
    const PlanHeader* hdr;
    const int4* light;
    const int4* chunks;
    const int4* heavy;
    float* part;
    int32_t part_stride;
    int32_t chunk_blocks;
    int32_t rows, edges;  // sizes the plan must have been built for
};

struct BwdParams {
    const void* qs;
    const void* ks;
    const void* v;
    const float* out;
    const float* lse;
    const float* dout;
    float* d_qs;
    float* d_ks;
    float* d_v;
    float* D;  // [N,H]
    BwdCsr a;  // by destination
    BwdCsr b;  // by source
    int32_t n, H, C, W, lpr_log2;
    int32_t own_rows;  // light rows: each edge group of a wavefront takes a row of its own
    float scale;      // dot: score scale
    float score_mul;  // multiplier taking a raw score to log2 units
    float slope;
    // kScoreAddEdge: the edge term of the logit and dz_e out, both in COO order [E, H],
    // reached through the COO index of each position of the CSR by destination (eid_a) and
    // by source (eid_b)
    const float* se;
    float* dz;
    const int32_t* eid_a;
    const int32_t* eid_b;
};

// Launchers, one per storage type (instantiated in local_bwd_f32.hip / local_bwd_bf16.hip).
bool launch_bwd_f32(const BwdParams& p, int epl, int hdp, int ns, int mode, unsigned grid_a, unsigned grid_b,
                    int64_t max_heavy, hipStream_t s);
bool launch_bwd_bf16(const BwdParams& p, int epl, int hdp, int ns, int mode, unsigned grid_a, unsigned grid_b,
                     int64_t max_heavy, hipStream_t s);

#ifdef GGA_BWD_IMPL

// ------------------------------------------------------------------------ pass A

// UMAX: edge slots per lane and iteration over the NS row slots (8 for rows that fill the
// wavefront, 4 for narrower rows, leaving registers for more resident wavefronts).
template <typename T, int EPL, int HDP, int NS, int MODE, int UMAX>
struct PassA {
    using V = Vec<T, EPL>;
    using raw_t = typename V::raw_t;
    static constexpr int kUMax = UMAX / NS;
    static constexpr int kAcc = MODE == GGA_SCORE_DOT ? EPL : 1;

    RowGeo<EPL, HDP, NS> geo;
    int U, EIT;
    float qf[NS][EPL], sd[NS], go[NS][EPL], Dh[NS], l2[NS];
    float acc[NS][kAcc];

    __device__ __forceinline__ void init(const BwdParams& p) {
        geo.init(p.lpr_log2, p.H, p.C);
        U = geo.G * kUMax <= 64 ? kUMax : 64 / geo.G;  // all slots, at most 64 edges per wave
        EIT = geo.G * U;
    }

    __device__ __forceinline__ void load_target(const BwdParams& p, int32_t v) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const size_t ro = (size_t)v * p.W + geo.off[s];
            float o[EPL];
            if (geo.ok[s]) {
                load_f32_once<EPL>(p.dout + ro, go[s]);
                load_f32_once<EPL>(p.out + ro, o);
            } else {
#pragma unroll
                for (int i = 0; i < EPL; i++) go[s][i] = o[i] = 0.f;
            }
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; i++) d = fmaf(go[s][i], o[i], d);
            Dh[s] = group_sum<HDP>(d);
            const size_t hi = (size_t)v * p.H + geo.head[s];
            l2[s] = geo.ok[s] ? p.lse[hi] * kLog2e : 0.f;
            if constexpr (MODE == GGA_SCORE_DOT) {
                raw_t r{};
                if (geo.ok[s]) r = load_once(reinterpret_cast<const raw_t*>(static_cast<const T*>(p.qs) + ro));
                V::widen(r, qf[s]);
            } else {
                sd[s] = geo.ok[s] ? static_cast<const float*>(p.qs)[hi] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < kAcc; i++) acc[s][i] = 0.f;
        }
    }

    // Shared row (OWN false): the groups take the edges beg + start + k*stride + (g + G*j).
    // Own rows (OWN true): group g alone takes beg + k*U + j of its own row, k < iters.
    template <bool OWN>
    __device__ __forceinline__ void run_t(const BwdParams& p, int32_t beg, int32_t end, int32_t start,
                                          int32_t stride, int32_t iters) {
        const T* __restrict__ kp = static_cast<const T*>(p.ks);
        const T* __restrict__ vp = static_cast<const T*>(p.v);
        const float* __restrict__ ssrc = static_cast<const float*>(p.ks);
        const int ll = OWN ? (geo.lane & (geo.lpr - 1)) : geo.lane;
        const int lim = OWN ? U : EIT;
        const int g0 = OWN ? geo.g * geo.lpr : 0;
        int32_t base = beg + start;
        int32_t colv = (ll < lim && base + ll < end) ? p.a.col[base + ll] : 0;
        int32_t eidv = 0;  // edge terms: the COO index of each position, loaded like col
        if constexpr (MODE == kScoreAddEdge) eidv = (ll < lim && base + ll < end) ? p.eid_a[base + ll] : 0;
        for (int32_t k = 0; OWN ? k < iters : base < end; k++, base += stride) {
            // the next iteration's sources, in flight while this iteration's rows are gathered
            const int32_t nxt = base + stride;
            const int32_t coln = (ll < lim && nxt + ll < end) ? p.a.col[nxt + ll] : 0;
            int32_t eidn = 0;
            if constexpr (MODE == kScoreAddEdge) eidn = (ll < lim && nxt + ll < end) ? p.eid_a[nxt + ll] : 0;
            int32_t u[kUMax], ej[kUMax];
            bool ev[kUMax];
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
                if (j < U) {
                    const int idx = OWN ? g0 + j : geo.g + geo.G * j;
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
                    if (ev[j] && geo.ok[s]) {
                        const size_t ro = (size_t)u[j] * p.W + geo.off[s];
                        if constexpr (MODE == GGA_SCORE_DOT) {
                            kr[j][s] = *reinterpret_cast<const raw_t*>(kp + ro);
                        } else {
                            ss[j][s] = ssrc[(size_t)u[j] * p.H + geo.head[s]];
                            if constexpr (MODE == kScoreAddEdge)
                                ss[j][s] += p.se[(size_t)ej[j] * p.H + geo.head[s]];
                        }
                        vr[j][s] = *reinterpret_cast<const raw_t*>(vp + ro);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
                if (j >= U) continue;
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    float vf[EPL];
                    V::widen(vr[j][s], vf);
                    float da = 0.f;
#pragma unroll
                    for (int i = 0; i < EPL; i++) da = fmaf(go[s][i], vf[i], da);
                    da = group_sum<HDP>(da);
                    if constexpr (MODE == GGA_SCORE_DOT) {
                        float kf[EPL];
                        V::widen(kr[j][s], kf);
                        float d = 0.f;
#pragma unroll
                        for (int i = 0; i < EPL; i++) d = fmaf(qf[s][i], kf[i], d);
                        d = group_sum<HDP>(d);
                        const float al = fexp2(d * p.score_mul - l2[s]);
                        const float ds = ev[j] ? al * (da - Dh[s]) * p.scale : 0.f;
#pragma unroll
                        for (int i = 0; i < EPL; i++) acc[s][i] = fmaf(ds, kf[i], acc[s][i]);
                    } else {
                        const float z = ss[j][s] + sd[s];
                        const float sc = (z > 0.f ? z : z * p.slope) * p.score_mul;
                        const float al = fexp2(sc - l2[s]);
                        const float ds = ev[j] ? al * (da - Dh[s]) : 0.f;
                        acc[s][0] = fmaf(ds, z > 0.f ? 1.f : p.slope, acc[s][0]);
                        if constexpr (MODE == kScoreAddEdge) {
                            if (ev[j] && geo.ok[s] && geo.lead[s])
                                p.dz[(size_t)ej[j] * p.H + geo.head[s]] =
                                    ds * (z > 0.f ? 1.f : p.slope);
                        }
                    }
                }
            }
            colv = coln;
            if constexpr (MODE == kScoreAddEdge) eidv = eidn;
        }
    }

    __device__ __forceinline__ void run(const BwdParams& p, int32_t beg, int32_t end, int32_t start,
                                        int32_t stride) {
        run_t<false>(p, beg, end, start, stride, 0);
    }

    __device__ __forceinline__ void reduce_groups() {
#pragma unroll
        for (int s = 0; s < NS; s++)
#pragma unroll
            for (int i = 0; i < kAcc; i++) acc[s][i] = sum_groups(acc[s][i], geo.lpr);
    }

    // Own rows: every group writes its own row v (one slot); nothing for `valid` false.
    // All 64 lanes must call it.
    __device__ __forceinline__ void write_own(const BwdParams& p, int32_t v, bool valid) {
        const size_t hi = (size_t)v * p.H + geo.head[0];
        if constexpr (MODE == GGA_SCORE_DOT) {
            if (geo.exact)
                store_group_row_nt<EPL>(p.d_qs + (size_t)v * p.W, acc[0], geo.lpr, geo.lane, valid);
            else if (valid && geo.ok[0])
                store_f32<EPL>(p.d_qs + (size_t)v * p.W + geo.off[0], acc[0]);
        } else {
            if (valid && geo.ok[0] && geo.lead[0]) p.d_qs[hi] = acc[0][0];
        }
        if (valid && geo.ok[0] && geo.lead[0]) p.D[hi] = Dh[0];
    }

    __device__ __forceinline__ void write_final(const BwdParams& p, int32_t v) {
        if constexpr (MODE == GGA_SCORE_DOT) {
            if (geo.exact) {  // all lanes take part (the row store exchanges chunks)
                store_row_nt<EPL>(p.d_qs + (size_t)v * p.W, acc[0], geo.lpr, geo.lane, geo.g);
                if (geo.g == 0 && geo.lead[0]) p.D[(size_t)v * p.H + geo.head[0]] = Dh[0];
                return;
            }
        }
        if (geo.g != 0) return;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (!geo.ok[s]) continue;
            const size_t hi = (size_t)v * p.H + geo.head[s];
            if constexpr (MODE == GGA_SCORE_DOT)
                store_f32<EPL>(p.d_qs + (size_t)v * p.W + geo.off[s], acc[s]);
            else if (geo.lead[s])
                p.d_qs[hi] = acc[s][0];
            if (geo.lead[s]) p.D[hi] = Dh[s];
        }
    }

    __device__ __forceinline__ void write_partial(const BwdParams& p, int32_t v, int32_t slot) {
        if (geo.g != 0) return;
        float* sp = p.a.part + (size_t)slot * p.a.part_stride;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (!geo.ok[s]) continue;
            if constexpr (MODE == GGA_SCORE_DOT)
                store_f32<EPL>(sp + geo.off[s], acc[s]);
            else if (geo.lead[s])
                sp[geo.head[s]] = acc[s][0];
            if (geo.lead[s]) p.D[(size_t)v * p.H + geo.head[s]] = Dh[s];
        }
    }
};

// ------------------------------------------------------------------------ pass B

template <typename T, int EPL, int HDP, int NS, int MODE>
struct PassB {
    using V = Vec<T, EPL>;
    using raw_t = typename V::raw_t;
    static constexpr int kUMax = 4 / NS;
    static constexpr int kAcc = MODE == GGA_SCORE_DOT ? EPL : 1;

    RowGeo<EPL, HDP, NS> geo;
    int U, EIT;
    float kf[NS][EPL], ssv[NS], vf[NS][EPL];
    float dk[NS][kAcc], dv[NS][EPL];

    __device__ __forceinline__ void init(const BwdParams& p) {
        geo.init(p.lpr_log2, p.H, p.C);
        U = geo.G * kUMax <= 64 ? kUMax : 64 / geo.G;  // all slots, at most 64 edges per wave
        EIT = geo.G * U;
    }

    __device__ __forceinline__ void load_source(const BwdParams& p, int32_t u) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const size_t ro = (size_t)u * p.W + geo.off[s];
            if constexpr (MODE != GGA_SCORE_MEAN) {
                raw_t r{};
                if (geo.ok[s]) r = load_once(reinterpret_cast<const raw_t*>(static_cast<const T*>(p.v) + ro));
                V::widen(r, vf[s]);
            }
            if constexpr (MODE == GGA_SCORE_DOT) {
                raw_t kr{};
                if (geo.ok[s]) kr = load_once(reinterpret_cast<const raw_t*>(static_cast<const T*>(p.ks) + ro));
                V::widen(kr, kf[s]);
            } else if constexpr (MODE != GGA_SCORE_MEAN) {
                ssv[s] = geo.ok[s] ? static_cast<const float*>(p.ks)[(size_t)u * p.H + geo.head[s]] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < kAcc; i++) dk[s][i] = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; i++) dv[s][i] = 0.f;
        }
    }

    // Shared row or own rows, as in pass A.
    template <bool OWN>
    __device__ __forceinline__ void run_t(const BwdParams& p, int32_t beg, int32_t end, int32_t start,
                                          int32_t stride, int32_t iters) {
        const T* __restrict__ qp = static_cast<const T*>(p.qs);
        const float* __restrict__ sdst = static_cast<const float*>(p.qs);
        const int ll = OWN ? (geo.lane & (geo.lpr - 1)) : geo.lane;
        const int lim = OWN ? U : EIT;
        const int g0 = OWN ? geo.g * geo.lpr : 0;
        int32_t base = beg + start;
        int32_t colv = (ll < lim && base + ll < end) ? p.b.col[base + ll] : 0;
        int32_t eidv = 0;  // edge terms: the COO index of each position, loaded like col
        if constexpr (MODE == kScoreAddEdge) eidv = (ll < lim && base + ll < end) ? p.eid_b[base + ll] : 0;
        for (int32_t k = 0; OWN ? k < iters : base < end; k++, base += stride) {
            // the next iteration's sources, in flight while this iteration's rows are gathered
            const int32_t nxt = base + stride;
            const int32_t coln = (ll < lim && nxt + ll < end) ? p.b.col[nxt + ll] : 0;
            int32_t eidn = 0;
            if constexpr (MODE == kScoreAddEdge) eidn = (ll < lim && nxt + ll < end) ? p.eid_b[nxt + ll] : 0;
            int32_t t[kUMax], ej[kUMax];
            bool ev[kUMax];
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
                if (j < U) {
                    const int idx = OWN ? g0 + j : geo.g + geo.G * j;
                    t[j] = __shfl(colv, idx, 64);
                    ej[j] = MODE == kScoreAddEdge ? __shfl(eidv, idx, 64) : 0;
                    ev[j] = base + (OWN ? j : idx) < end;
                } else {
                    t[j] = 0;
                    ej[j] = 0;
                    ev[j] = false;
                }
            }
            raw_t qr[kUMax][NS];
            float gr[kUMax][NS][EPL];
            float lj[kUMax][NS], dj[kUMax][NS], sj[kUMax][NS];
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    qr[j][s] = raw_t{};
                    lj[j][s] = dj[j][s] = sj[j][s] = 0.f;
#pragma unroll
                    for (int i = 0; i < EPL; i++) gr[j][s][i] = 0.f;
                    if (ev[j] && geo.ok[s]) {
                        const size_t ro = (size_t)t[j] * p.W + geo.off[s];
                        const size_t hi = (size_t)t[j] * p.H + geo.head[s];
                        if constexpr (MODE == GGA_SCORE_DOT) {
                            qr[j][s] = *reinterpret_cast<const raw_t*>(qp + ro);
                        } else if constexpr (MODE != GGA_SCORE_MEAN) {
                            sj[j][s] = sdst[hi];
                            if constexpr (MODE == kScoreAddEdge)
                                sj[j][s] += p.se[(size_t)ej[j] * p.H + geo.head[s]];
                        }
                        load_f32<EPL>(p.dout + ro, gr[j][s]);
                        if constexpr (MODE == GGA_SCORE_MEAN) {  // the weight itself: 1/deg(t)
                            lj[j][s] = 1.f / (float)(p.a.row_ptr[t[j] + 1] - p.a.row_ptr[t[j]]);
                        } else {
                            lj[j][s] = p.lse[hi];
                            dj[j][s] = p.D[hi];
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kUMax; j++) {
                if (j >= U) continue;
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    if constexpr (MODE == GGA_SCORE_MEAN) {
                        const float al = ev[j] ? lj[j][s] : 0.f;
#pragma unroll
                        for (int i = 0; i < EPL; i++) dv[s][i] = fmaf(al, gr[j][s][i], dv[s][i]);
                        continue;
                    }
                    float da = 0.f;
#pragma unroll
                    for (int i = 0; i < EPL; i++) da = fmaf(gr[j][s][i], vf[s][i], da);
                    da = group_sum<HDP>(da);
                    float al, ds;
                    if constexpr (MODE == GGA_SCORE_DOT) {
                        float qf[EPL];
                        V::widen(qr[j][s], qf);
                        float d = 0.f;
#pragma unroll
                        for (int i = 0; i < EPL; i++) d = fmaf(qf[i], kf[s][i], d);
                        d = group_sum<HDP>(d);
                        al = ev[j] ? fexp2(d * p.score_mul - lj[j][s] * kLog2e) : 0.f;
                        ds = al * (da - dj[j][s]) * p.scale;
#pragma unroll
                        for (int i = 0; i < EPL; i++) dk[s][i] = fmaf(ds, qf[i], dk[s][i]);
                    } else {
                        const float z = ssv[s] + sj[j][s];
                        const float sc = (z > 0.f ? z : z * p.slope) * p.score_mul;
                        al = ev[j] ? fexp2(sc - lj[j][s] * kLog2e) : 0.f;
                        ds = al * (da - dj[j][s]);
                        dk[s][0] = fmaf(ds, z > 0.f ? 1.f : p.slope, dk[s][0]);
                    }
#pragma unroll
                    for (int i = 0; i < EPL; i++) dv[s][i] = fmaf(al, gr[j][s][i], dv[s][i]);
                }
            }
            colv = coln;
            if constexpr (MODE == kScoreAddEdge) eidv = eidn;
        }
    }

    __device__ __forceinline__ void run(const BwdParams& p, int32_t beg, int32_t end, int32_t start,
                                        int32_t stride) {
        run_t<false>(p, beg, end, start, stride, 0);
    }

    // Own rows: every group writes its own row u (one slot); nothing for `valid` false.
    // All 64 lanes must call it.
    __device__ __forceinline__ void write_own(const BwdParams& p, int32_t u, bool valid) {
        if (geo.exact) {
            if constexpr (MODE == GGA_SCORE_DOT)
                store_group_row_nt<EPL>(p.d_ks + (size_t)u * p.W, dk[0], geo.lpr, geo.lane, valid);
            else if constexpr (MODE != GGA_SCORE_MEAN)
                if (valid && geo.lead[0]) p.d_ks[(size_t)u * p.H + geo.head[0]] = dk[0][0];
            store_group_row_nt<EPL>(p.d_v + (size_t)u * p.W, dv[0], geo.lpr, geo.lane, valid);
            return;
        }
        if (!valid || !geo.ok[0]) return;
        if constexpr (MODE == GGA_SCORE_DOT)
            store_f32<EPL>(p.d_ks + (size_t)u * p.W + geo.off[0], dk[0]);
        else if constexpr (MODE != GGA_SCORE_MEAN)
            if (geo.lead[0]) p.d_ks[(size_t)u * p.H + geo.head[0]] = dk[0][0];
        store_f32<EPL>(p.d_v + (size_t)u * p.W + geo.off[0], dv[0]);
    }

    __device__ __forceinline__ void reduce_groups() {
#pragma unroll
        for (int s = 0; s < NS; s++) {
#pragma unroll
            for (int i = 0; i < kAcc; i++) dk[s][i] = sum_groups(dk[s][i], geo.lpr);
#pragma unroll
            for (int i = 0; i < EPL; i++) dv[s][i] = sum_groups(dv[s][i], geo.lpr);
        }
    }

    __device__ __forceinline__ int dk_width(const BwdParams& p) const {
        return MODE == GGA_SCORE_DOT ? p.W : MODE == GGA_SCORE_MEAN ? 0 : p.H;
    }

    __device__ __forceinline__ void write_to(const BwdParams& p, float* dkp, float* dvp) {
        if (geo.g != 0) return;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (!geo.ok[s]) continue;
            if constexpr (MODE == GGA_SCORE_DOT)
                store_f32<EPL>(dkp + geo.off[s], dk[s]);
            else if (MODE != GGA_SCORE_MEAN && geo.lead[s])
                dkp[geo.head[s]] = dk[s][0];
            store_f32<EPL>(dvp + geo.off[s], dv[s]);
        }
    }

    __device__ __forceinline__ void write_final(const BwdParams& p, int32_t u) {
        if (geo.exact) {  // all lanes take part (the row store exchanges chunks)
            if constexpr (MODE == GGA_SCORE_DOT) {
                store_row_nt<EPL>(p.d_ks + (size_t)u * p.W, dk[0], geo.lpr, geo.lane, geo.g);
            } else if constexpr (MODE != GGA_SCORE_MEAN) {
                if (geo.g == 0 && geo.lead[0]) p.d_ks[(size_t)u * p.H + geo.head[0]] = dk[0][0];
            }
            store_row_nt<EPL>(p.d_v + (size_t)u * p.W, dv[0], geo.lpr, geo.lane, geo.g);
            return;
        }
        write_to(p, MODE == GGA_SCORE_MEAN ? nullptr : p.d_ks + (size_t)u * dk_width(p), p.d_v + (size_t)u * p.W);
    }

    __device__ __forceinline__ void write_partial(const BwdParams& p, int32_t slot) {
        float* sp = p.b.part + (size_t)slot * p.b.part_stride;
        write_to(p, sp, sp + align8(dk_width(p)));
    }

    __device__ __forceinline__ static int align8(int x) { return (x + 7) & ~7; }
};

// ------------------------------------------------------------------------ kernels

// Iterations of U edges that the longest of a wavefront's own rows needs (deg: this
// group's row length; the result is the same in every lane).
__device__ __forceinline__ int32_t own_iters(int32_t deg, int U, int lpr) {
    int32_t it = (deg + U - 1) / U;
    for (int o = lpr; o < 64; o <<= 1) it = max(it, __shfl_xor(it, o, 64));
    return it;
}

// Adds the per-wave partial arrays of a workgroup through LDS in wave order.
template <int N>
__device__ __forceinline__ void lds_sum_waves(float (&x)[N], float (*sm)[64][N], int wave, int lane) {
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < N; i++) sm[wave][lane][i] = x[i];
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 1; w < kBwdWaves; w++)
#pragma unroll
            for (int i = 0; i < N; i++) x[i] += sm[w][lane][i];
    }
}

template <typename T, int EPL, int HDP, int NS, int MODE, int UMAX>
__global__ __launch_bounds__(kBwdThreads) void bwd_dst_kernel(BwdParams p) {
    using Row = PassA<T, EPL, HDP, NS, MODE, UMAX>;
    constexpr int kA = Row::kAcc;
    if (!plan_usable(p.a.hdr, p.a.rows, p.a.edges)) return;
    Row r;
    r.init(p);
    const int wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < p.a.chunk_blocks) {
        __shared__ float sm[kBwdWaves][64][NS * kA];
        const int nch = p.a.hdr->n_chunks;
        for (int c = blockIdx.x; c < nch; c += p.a.chunk_blocks) {
            const int4 ch = p.a.chunks[c];
            r.load_target(p, ch.x);
            r.run(p, ch.y, ch.z, wave * r.EIT, kBwdWaves * r.EIT);
            r.reduce_groups();
            float flat[NS * kA];
#pragma unroll
            for (int s = 0; s < NS; s++)
#pragma unroll
                for (int i = 0; i < kA; i++) flat[s * kA + i] = r.acc[s][i];
            lds_sum_waves<NS * kA>(flat, sm, wave, r.geo.lane);
            if (wave == 0) {
#pragma unroll
                for (int s = 0; s < NS; s++)
#pragma unroll
                    for (int i = 0; i < kA; i++) r.acc[s][i] = flat[s * kA + i];
                if (ch.w < 0)
                    r.write_final(p, ch.x);
                else
                    r.write_partial(p, ch.x, ch.w);
            }
            __syncthreads();
        }
        return;
    }
    const int nl = p.a.hdr->n_light;
    if (NS == 1 && UMAX == 4 && p.own_rows) {  // the wavefront owns G consecutive light rows
        const int li0 = ((blockIdx.x - p.a.chunk_blocks) * kBwdWaves + wave) * r.geo.G;
        if (li0 >= nl) return;
        if ((int64_t)p.a.hdr->light_sum > (int64_t)nl * r.EIT) {  // long rows: one after another
            const int lend = min(li0 + r.geo.G, nl);
            for (int li = li0; li < lend; li++) {
                const int4 lr = p.a.light[li];
                r.load_target(p, lr.x);
                r.run(p, lr.y, lr.z, 0, r.EIT);
                r.reduce_groups();
                r.write_final(p, lr.x);
            }
            return;
        }
        const int li = li0 + r.geo.g;  // short rows: each group takes one
        const bool valid = li < nl;
        const int4 lr = valid ? p.a.light[li] : make_int4(0, 0, 0, 0);
        const int32_t iters = own_iters(lr.z - lr.y, r.U, r.geo.lpr);
        r.load_target(p, lr.x);
        r.template run_t<true>(p, lr.y, lr.z, 0, r.U, iters);
        r.write_own(p, lr.x, valid);
        return;
    }
    const int li = (blockIdx.x - p.a.chunk_blocks) * kBwdWaves + wave;
    if (li >= nl) return;
    const int4 lr = p.a.light[li];
    const int32_t v = lr.x;
    r.load_target(p, v);
    r.run(p, lr.y, lr.z, 0, r.EIT);
    r.reduce_groups();
    r.write_final(p, v);
}

template <typename T, int EPL, int HDP, int NS, int MODE>
__global__ __launch_bounds__(kBwdThreads) void bwd_src_kernel(BwdParams p) {
    using Row = PassB<T, EPL, HDP, NS, MODE>;
    constexpr int kA = Row::kAcc;
    constexpr int kF = NS * (kA + EPL);
    if (!plan_usable(p.b.hdr, p.b.rows, p.b.edges)) return;
    Row r;
    r.init(p);
    const int wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < p.b.chunk_blocks) {
        __shared__ float sm[kBwdWaves][64][kF];
        const int nch = p.b.hdr->n_chunks;
        for (int c = blockIdx.x; c < nch; c += p.b.chunk_blocks) {
            const int4 ch = p.b.chunks[c];
            r.load_source(p, ch.x);
            r.run(p, ch.y, ch.z, wave * r.EIT, kBwdWaves * r.EIT);
            r.reduce_groups();
            float flat[kF];
#pragma unroll
            for (int s = 0; s < NS; s++) {
#pragma unroll
                for (int i = 0; i < kA; i++) flat[s * (kA + EPL) + i] = r.dk[s][i];
#pragma unroll
                for (int i = 0; i < EPL; i++) flat[s * (kA + EPL) + kA + i] = r.dv[s][i];
            }
            lds_sum_waves<kF>(flat, sm, wave, r.geo.lane);
            if (wave == 0) {
#pragma unroll
                for (int s = 0; s < NS; s++) {
#pragma unroll
                    for (int i = 0; i < kA; i++) r.dk[s][i] = flat[s * (kA + EPL) + i];
#pragma unroll
                    for (int i = 0; i < EPL; i++) r.dv[s][i] = flat[s * (kA + EPL) + kA + i];
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
    const int nl = p.b.hdr->n_light;
    if (NS == 1 && p.own_rows) {  // the wavefront owns G consecutive light rows
        const int li0 = ((blockIdx.x - p.b.chunk_blocks) * kBwdWaves + wave) * r.geo.G;
        if (li0 >= nl) return;
        if ((int64_t)p.b.hdr->light_sum > (int64_t)nl * r.EIT) {  // long rows: one after another
            const int lend = min(li0 + r.geo.G, nl);
            for (int li = li0; li < lend; li++) {
                const int4 lr = p.b.light[li];
                r.load_source(p, lr.x);
                r.run(p, lr.y, lr.z, 0, r.EIT);
                r.reduce_groups();
                r.write_final(p, lr.x);
            }
            return;
        }
        const int li = li0 + r.geo.g;  // short rows: each group takes one
        const bool valid = li < nl;
        const int4 lr = valid ? p.b.light[li] : make_int4(0, 0, 0, 0);
        const int32_t iters = own_iters(lr.z - lr.y, r.U, r.geo.lpr);
        r.load_source(p, lr.x);
        r.template run_t<true>(p, lr.y, lr.z, 0, r.U, iters);
        r.write_own(p, lr.x, valid);
        return;
    }
    const int li = (blockIdx.x - p.b.chunk_blocks) * kBwdWaves + wave;
    if (li >= nl) return;
    const int4 lr = p.b.light[li];
    const int32_t u = lr.x;
    r.load_source(p, u);
    r.run(p, lr.y, lr.z, 0, r.EIT);
    r.reduce_groups();
    r.write_final(p, u);
}

// Adds the partial sums of each split row in slot order: `width` leading values go to
// out_a (row stride width), and, when width_b > 0, the next width_b values (starting at
// the 8-aligned offset) go to out_b.
static __global__ __launch_bounds__(kBwdThreads) void bwd_merge(BwdCsr c, int width, float* out_a, int width_b,
                                                         float* out_b) {
    if (!plan_usable(c.hdr, c.rows, c.edges)) return;
    const int lane = threadIdx.x & 63;
    const int nh = c.hdr->n_heavy;
    const int off_b = (width + 7) & ~7;
    for (int hr = blockIdx.x * kBwdWaves + (threadIdx.x >> 6); hr < nh; hr += gridDim.x * kBwdWaves) {
        const int4 hv = c.heavy[hr];
        for (int x = lane; x < width + width_b; x += 64) {
            const int col = x < width ? x : off_b + (x - width);
            float a = 0.f;
            for (int i0 = 0; i0 < hv.z; i0 += 8) {  // eight slots' loads in flight, added in slot order
                float t[8];
#pragma unroll
                for (int j = 0; j < 8; j++) t[j] = i0 + j < hv.z ? c.part[(size_t)(hv.y + i0 + j) * c.part_stride + col] : 0.f;
#pragma unroll
                for (int j = 0; j < 8; j++)
                    if (i0 + j < hv.z) a += t[j];
            }
            if (x < width)
                out_a[(size_t)hv.x * width + x] = a;
            else
                out_b[(size_t)hv.x * width_b + (x - width)] = a;
        }
    }
}

template <typename T, int EPL, int HDP, int NS, int MODE, int UMAX>
void launch_bwd_t(const BwdParams& p, unsigned grid_a, unsigned grid_b, int64_t max_heavy, hipStream_t s) {
    const int wk = MODE == GGA_SCORE_DOT ? p.W : MODE == GGA_SCORE_MEAN ? 0 : p.H;
    int64_t mb = (max_heavy + kBwdWaves - 1) / kBwdWaves;
    const unsigned mg = (unsigned)(mb < 1024 ? (mb < 1 ? 1 : mb) : 1024);
    if constexpr (MODE != GGA_SCORE_MEAN) {
        bwd_dst_kernel<T, EPL, HDP, NS, MODE, UMAX><<<grid_a, kBwdThreads, 0, s>>>(p);
        if (max_heavy > 0) bwd_merge<<<mg, kBwdThreads, 0, s>>>(p.a, wk, p.d_qs, 0, nullptr);
    }
    bwd_src_kernel<T, EPL, HDP, NS, MODE><<<grid_b, kBwdThreads, 0, s>>>(p);
    if (max_heavy > 0) bwd_merge<<<mg, kBwdThreads, 0, s>>>(p.b, wk, p.d_ks, p.W, p.d_v);
}

template <typename T, int EPL, int MODE>
bool launch_bwd_hdp(const BwdParams& p, int hdp, int ns, unsigned ga, unsigned gb, int64_t mh, hipStream_t s) {
#define GGA_BCASE(HD)                                                 \
    case HD:                                                          \
        if (ns == 1 && p.lpr_log2 == 6)                               \
            launch_bwd_t<T, EPL, HD, 1, MODE, 8>(p, ga, gb, mh, s);   \
        else if (ns == 1)                                             \
            launch_bwd_t<T, EPL, HD, 1, MODE, 4>(p, ga, gb, mh, s);   \
        else if constexpr (EPL > 1)                                   \
            launch_bwd_t<T, EPL, HD, 2, MODE, 8>(p, ga, gb, mh, s);   \
        else                                                        \
            return false;                                           \
        return true;
    switch (hdp) {
        GGA_BCASE(1)
        GGA_BCASE(2)
        GGA_BCASE(4)
        GGA_BCASE(8)
        GGA_BCASE(16)
        GGA_BCASE(32)
        GGA_BCASE(64)
        default:
            return false;
    }
#undef GGA_BCASE
}

template <typename T, int VEC>
bool launch_bwd_dtype(const BwdParams& p, int epl, int hdp, int ns, int mode, unsigned ga, unsigned gb,
                      int64_t mh, hipStream_t s) {
    if (mode == GGA_SCORE_DOT) {
        if (epl == VEC) return launch_bwd_hdp<T, VEC, GGA_SCORE_DOT>(p, hdp, ns, ga, gb, mh, s);
        return launch_bwd_hdp<T, 1, GGA_SCORE_DOT>(p, hdp, ns, ga, gb, mh, s);
    }
    if (mode == GGA_SCORE_MEAN) {
        if (epl == VEC) return launch_bwd_hdp<T, VEC, GGA_SCORE_MEAN>(p, hdp, ns, ga, gb, mh, s);
        return launch_bwd_hdp<T, 1, GGA_SCORE_MEAN>(p, hdp, ns, ga, gb, mh, s);
    }
    if (mode == kScoreAddEdge) {  // fp32 node tensors only
        if constexpr (std::is_same<T, float>::value) {
            if (epl == VEC) return launch_bwd_hdp<T, VEC, kScoreAddEdge>(p, hdp, ns, ga, gb, mh, s);
            return launch_bwd_hdp<T, 1, kScoreAddEdge>(p, hdp, ns, ga, gb, mh, s);
        }
        return false;
    }
    if (epl == VEC) return launch_bwd_hdp<T, VEC, GGA_SCORE_ADDITIVE>(p, hdp, ns, ga, gb, mh, s);
    return launch_bwd_hdp<T, 1, GGA_SCORE_ADDITIVE>(p, hdp, ns, ga, gb, mh, s);
}

#endif  // GGA_BWD_IMPL

}  // namespace gga
