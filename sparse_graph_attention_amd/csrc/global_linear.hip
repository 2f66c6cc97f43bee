// Global linear-attention branch ("Gated Local-Global Graph Attention", Key formulas G_i,
// S, z; Implementation notes item 2, phi = elu + 1), forward and backward, per graph b and
// head h of width r:
//   S[b,h] = sum_{j in b} phi(k_j) v_j^T,  z[b,h] = sum_{j in b} phi(k_j),
//   G[i] = phi(q_i)^T S[b,h] / (phi(q_i) . z[b,h] + eps)      (i in graph b).
// One graph is the plain layer; several graphs packed along the node axis are the batched
// input of the page's Implementation notes (one adjacency list per graph).
//
// Work is cut into tiles of `rs` consecutive node rows (rs a multiple of 16, at least 256,
// fixed by n and the head count, so at most 1024 / heads tiles and 1024 tiles x heads).  A graph of at most rs rows is handled whole by the
// tile holding its first row; a longer graph is cut at tile boundaries and each piece gives
// a partial sum in one of two slots of its tile (slot 0: the graph holding the tile's first
// row; slot 1: a long graph starting inside the tile), which a second kernel adds in tile
// order.  Every sum therefore has a fixed order.  For r a multiple of 16 (up to 64) the
// contractions run on the matrix cores (v_mfma_f32_16x16x4_f32); other widths take scalar
// paths.
#include "common.hpp"

namespace gga {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// d phi / dx given x and phi(x): 1 for x > 0, e^x = phi(x) otherwise
__device__ __forceinline__ float dphi(float x, float p) { return x > 0.f ? 1.f : p; }

// N consecutive floats (N = 1..4) in one access; p must be 4*N-byte aligned (16 for N = 3).
template <int N>
__device__ __forceinline__ void load_n(const float* p, float* out) {
    if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        out[0] = t.x; out[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = p[i];
    }
}

template <int N>
__device__ __forceinline__ void store_n(float* p, const float* v) {
    if constexpr (N == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) p[i] = v[i];
    }
}

// ---------------------------------------------------------------- graphs and tiles

struct Seg {
    const int32_t* node_ptr;  // [batch + 1]; nullptr: one graph of n rows
    int32_t batch;
    int32_t n;
    int32_t rs;  // rows per tile

    // first row of graph b, clamped to [0, n] (so a malformed node_ptr cannot send an
    // access out of bounds)
    __device__ __forceinline__ int64_t node(int32_t b) const {
        const int64_t v = node_ptr ? node_ptr[b] : (b == 0 ? 0 : n);
        return v < 0 ? 0 : (v > n ? n : v);
    }
    // the graph holding `row`: the last b with node(b) <= row, clamped to [0, batch)
    __device__ __forceinline__ int32_t graph_of(int64_t row) const {
        if (!node_ptr) return 0;
        int32_t lo = 0, hi = batch + 1;
        while (lo < hi) {
            const int32_t mid = (lo + hi) >> 1;
            if (node(mid) <= row)
                lo = mid + 1;
            else
                hi = mid;
        }
        const int32_t b = lo - 1;
        return b < 0 ? 0 : (b >= batch ? batch - 1 : b);
    }
};

struct Piece {
    int32_t b;
    int64_t r0, r1;
    int slot;
};

// The pieces of tile t in order, one per call of next(): the first test covers a long graph
// that began before (or at) the tile's first row, the loop the graphs starting inside it.
struct PieceIter {
    const Seg& sg;
    int64_t a, e;
    int32_t b;
    bool first;
    __device__ __forceinline__ PieceIter(const Seg& s, int64_t t) : sg(s), first(true) {
        a = t * sg.rs;
        e = a + sg.rs < sg.n ? a + sg.rs : sg.n;
        b = a < e ? sg.graph_of(a) : sg.batch;
    }
    __device__ __forceinline__ bool next(Piece& p) {
        if (a >= e) return false;
        if (first) {
            first = false;
            const int64_t lo = sg.node(b), hi = sg.node(b + 1);
            if (lo <= a && a < hi) {
                if (hi - lo > sg.rs) {
                    p = Piece{b, a, hi < e ? hi : e, 0};
                    b++;
                    return true;
                }
                if (lo < a) b++;  // a short graph that started in an earlier tile
            }
        }
        for (; b < sg.batch; b++) {
            const int64_t lo = sg.node(b), hi = sg.node(b + 1);
            if (lo >= e) return false;
            if (lo < a || hi <= lo) continue;
            p = hi - lo > sg.rs ? Piece{b, lo, hi < e ? hi : e, 1} : Piece{b, lo, hi, -1};
            b++;
            return true;
        }
        return false;
    }
};

// Calls f(b, r0, r1, slot) for the pieces tile t handles, in graph order: slot 0 or 1 for a
// piece of a long graph (rows of the tile), -1 for a whole short graph (its rows may run
// past the tile).  Depends only on t, so it is uniform across a workgroup.  One call site,
// so f's body is compiled once.
template <class F>
__device__ __forceinline__ void for_each_segment(const Seg& sg, int64_t t, F&& f) {
    PieceIter it(sg, t);
    Piece p;
    while (it.next(p)) f(p.b, p.r0, p.r1, p.slot);
}

// The long graph whose first row lies in tile t, or -1.
__device__ __forceinline__ int32_t owned_long(const Seg& sg, int64_t t, int64_t& lo, int64_t& hi) {
    const int64_t a = t * sg.rs;
    const int64_t e = a + sg.rs < sg.n ? a + sg.rs : sg.n;
    if (a >= e) return -1;
    const int32_t b = sg.graph_of(e - 1);
    lo = sg.node(b);
    hi = sg.node(b + 1);
    return (lo >= a && lo < e && hi - lo > sg.rs) ? b : -1;
}

// The long graphs in the order of their first tiles: list[0 .. *count) = (first tile,
// graph, first row, end row).  One workgroup of 1024 threads; there are at most 1024 tiles.
__global__ __launch_bounds__(1024) void list_long(Seg sg, int64_t tiles, int4* __restrict__ list,
                                                  int32_t* __restrict__ count) {
    __shared__ int wsum[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t lo = 0, hi = 0;
    const int32_t b = t < tiles ? owned_long(sg, t, lo, hi) : -1;
    const int flag = b >= 0 ? 1 : 0;
    int x = flag;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; w++) before += wsum[w];
    if (flag) list[before + x - 1] = make_int4(t, b, (int)lo, (int)hi);
    if (t == 1023) count[0] = before + x;
}

// ---------------------------------------------------------------- statistics

template <int TR>
__device__ __forceinline__ void store_stats(float* sdst, float* zdst, const v4f (&acc)[TR][TR],
                                            const float (&zacc)[TR], int lane) {
    constexpr int R = TR * 16;
    // acc[i][j][q] of lane l is S[TR*pi + i][TR*pj + j] with pi = (l/16)*4 + q, pj = l%16
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int pi = (lane >> 4) * 4 + q, pj = lane & 15;
#pragma unroll
        for (int i = 0; i < TR; i++) {
            float row[TR];
#pragma unroll
            for (int j = 0; j < TR; j++) row[j] = acc[i][j][q];
            store_n<TR>(sdst + (TR * pi + i) * R + TR * pj, row);
        }
    }
    if (lane < 16) store_n<TR>(zdst + TR * lane, zacc);
}

// Matrix-core path.  grid (tiles); one wavefront per head (up to 8; more heads loop), so
// the wavefronts of a workgroup read the same rows.  Each step takes 4 rows (lane / 16);
// four steps are loaded before any is multiplied.  Feature order inside a head is permuted:
// MFMA tile u, position p <-> feature TR*p + u, so lane p loads its TR features of a row as
// one vector.
template <int TR>
__global__ __launch_bounds__(512) void stats_mfma(Seg sg, int32_t H, const float* __restrict__ k,
                                                   const float* __restrict__ v, float* __restrict__ part,
                                                   float* __restrict__ s, float* __restrict__ z) {
    constexpr int R = TR * 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int64_t W = (int64_t)H * R;
    const int64_t t = blockIdx.x;
    for_each_segment(sg, t, [&](int32_t b, int64_t r0, int64_t r1, int slot) {
        for (int h = wave; h < H; h += nw) {
            v4f acc[TR][TR];
            float zacc[TR];
#pragma unroll
            for (int i = 0; i < TR; i++) {
                zacc[i] = 0.f;
#pragma unroll
                for (int j = 0; j < TR; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
            // the next 16 rows are loaded during the current rows' MFMAs; rows past the piece
            // read its last row and are zeroed by a select, so no load is conditional
            float kn[4][TR], vn[4][TR];
            auto fetch = [&](int64_t base) {
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    const int64_t row = base + st * 4 + (lane >> 4);
                    const int64_t o = (row < r1 ? row : r1 - 1) * W + h * R + TR * (lane & 15);
                    load_n<TR>(k + o, kn[st]);
                    load_n<TR>(v + o, vn[st]);
                }
            };
            if (r0 < r1) fetch(r0);
            for (int64_t base = r0; base < r1; base += 16) {
                float a[4][TR], bv[4][TR];
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    const bool ok = base + st * 4 + (lane >> 4) < r1;
#pragma unroll
                    for (int u = 0; u < TR; u++) {
                        a[st][u] = ok ? phi(kn[st][u]) : 0.f;
                        bv[st][u] = ok ? vn[st][u] : 0.f;
                    }
                }
                if (base + 16 < r1) fetch(base + 16);
#pragma unroll
                for (int st = 0; st < 4; st++) {
#pragma unroll
                    for (int u = 0; u < TR; u++) zacc[u] += a[st][u];
#pragma unroll
                    for (int i = 0; i < TR; i++)
#pragma unroll
                        for (int j = 0; j < TR; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st][i], bv[st][j], acc[i][j], 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < TR; u++) {
                zacc[u] += __shfl_xor(zacc[u], 16, 64);
                zacc[u] += __shfl_xor(zacc[u], 32, 64);
            }
            if (slot < 0) {
                store_stats<TR>(s + ((int64_t)b * H + h) * R * R, z + ((int64_t)b * H + h) * R, acc, zacc, lane);
            } else {
                float* out = part + ((t * 2 + slot) * H + h) * (R * R + R);
                store_stats<TR>(out, out + R * R, acc, zacc, lane);
            }
        }
    });
}

// Scalar path (any r).  grid (tiles, H); threads over the r*r + r outputs.
__global__ __launch_bounds__(256) void stats_scalar(Seg sg, int32_t H, int32_t R, const float* __restrict__ k,
                                                    const float* __restrict__ v, float* __restrict__ part,
                                                    float* __restrict__ s, float* __restrict__ z) {
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t t = blockIdx.x;
    for_each_segment(sg, t, [&](int32_t b, int64_t r0, int64_t r1, int slot) {
        for (int e = threadIdx.x; e < R * R + R; e += blockDim.x) {
            float acc = 0.f;
            if (e < R * R) {
                const int i = e / R, j = e % R;
                for (int64_t row = r0; row < r1; row++)
                    acc = fmaf(phi(k[row * W + h * R + i]), v[row * W + h * R + j], acc);
            } else {
                const int i = e - R * R;
                for (int64_t row = r0; row < r1; row++) acc += phi(k[row * W + h * R + i]);
            }
            if (slot >= 0)
                part[((t * 2 + slot) * H + h) * (R * R + R) + e] = acc;
            else if (e < R * R)
                s[((int64_t)b * H + h) * R * R + e] = acc;
            else
                z[((int64_t)b * H + h) * R + e - R * R] = acc;
        }
    });
}

// Adds the pieces of each long graph in tile order.  grid (ceil(H*(r*r+r)/64), L): a
// workgroup of NW wavefronts owns 64 consecutive outputs of the graphs list[y], y =
// blockIdx.y, blockIdx.y + L, ...; wavefront w adds tiles w, w+NW, ... of the graph and the
// NW sums are added in wavefront order.
template <int NW>
__global__ __launch_bounds__(NW * 64) void seg_reduce(Seg sg, int32_t H, int32_t R, const int4* __restrict__ list,
                                                      const int32_t* __restrict__ count,
                                                      const float* __restrict__ part, float* __restrict__ s,
                                                      float* __restrict__ z) {
    __shared__ float sm[NW][64];
    const int per = R * R + R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t x = (int64_t)blockIdx.x * 64 + lane;
    const int64_t tot = (int64_t)H * per;
    const int h = (int)(x / per), e = (int)(x % per);
    const int nl = count[0];
    for (int y = blockIdx.y; y < nl; y += gridDim.y) {
        const int4 ent = list[y];
        const int64_t t0 = ent.x, lo = ent.z, hi = ent.w;
        const int32_t b = ent.y;
        const int64_t t1 = (hi - 1) / sg.rs;
        float a = 0.f;
        if (x < tot) {
            // eight of the wavefront's tiles are requested at a time and added in tile order
            int64_t tt = t0 + wave;
            for (; tt + 7 * NW <= t1; tt += 8 * NW) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const int64_t u = tt + (int64_t)j * NW;
                    const int slot = (u == t0 && lo != t0 * sg.rs) ? 1 : 0;
                    v[j] = part[((u * 2 + slot) * H + h) * per + e];
                }
#pragma unroll
                for (int j = 0; j < 8; j++) a += v[j];
            }
            for (; tt <= t1; tt += NW) {
                const int slot = (tt == t0 && lo != t0 * sg.rs) ? 1 : 0;
                a += part[((tt * 2 + slot) * H + h) * per + e];
            }
        }
        __syncthreads();
        sm[wave][lane] = a;
        __syncthreads();
        if (wave == 0 && x < tot) {
            float acc = 0.f;
            for (int w = 0; w < NW; w++) acc += sm[w][lane];
            if (e < R * R)
                s[((int64_t)b * H + h) * R * R + e] = acc;
            else
                z[((int64_t)b * H + h) * R + e - R * R] = acc;
        }
    }
}

// ---------------------------------------------------------------- G = phi(Q) S / (phi(Q) z + eps)

// Lane layout of the row passes (apply_mfma and the two backward passes): lane group
// gq = lane / 16 of row li = lane % 16 holds, as its t-th value (t = 4c + e), feature
// feat(gq, t) = 16c + 4gq + e of the head, so the c-th 16-byte load or store of the four
// groups covers 64 contiguous bytes of the row (one memory request, not four 16-byte ones
// 64 bytes apart).  An MFMA output tile j covers features 16j .. 16j+15 of which group gq
// holds positions 4gq .. 4gq+3, the same features as its t = 4j .. 4j+3: inputs and outputs
// of a lane line up.
__device__ __forceinline__ int feat(int gq, int t) { return 16 * (t >> 2) + 4 * gq + (t & 3); }

// N consecutive floats from LDS as one vector read where N allows.
template <int N>
__device__ __forceinline__ void lds_load_n(const float* p, float* out) {
    if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        out[0] = t.x; out[1] = t.y; out[2] = t.z; out[3] = t.w;
    } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        out[0] = t.x; out[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = p[i];
    }
}

// Matrix-core path.  grid (tiles, H), four wavefronts on head blockIdx.y; the piece's S and z
// sit in LDS and the wavefronts take its 16-row tiles in turn.  The contraction index follows
// feat: in MFMA step t the lane group gq = lane/16 supplies k = feat(gq, t), so each lane's A
// operands over the R/4 steps come from 16-byte loads that together read 64 contiguous bytes
// of the row; its B operands S[k][TR*li .. TR*li+TR-1] are one LDS vector per step.  Output
// columns are permuted too (MFMA tile j, position li <-> column TR*li + j), so each lane ends
// with TR consecutive outputs of a row.  The next tile's q is loaded (and kept raw until
// used) before the current one is multiplied.  (S held in registers for a whole piece took
// 256 registers: two wavefronts per SIMD, each with one tile's loads in flight.)
template <int TR>
__global__ __launch_bounds__(256) void apply_mfma(Seg sg, int32_t H, float eps, const float* __restrict__ q,
                                                   const float* __restrict__ s, const float* __restrict__ z,
                                                   float* __restrict__ g) {
    constexpr int R = TR * 16;
    constexpr int KQ = R / 4;  // MFMA steps per row tile
    __shared__ __align__(16) float sl[R * R], zl[R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    for_each_segment(sg, blockIdx.x, [&](int32_t b, int64_t r0, int64_t r1, int) {
        const int64_t bh = (int64_t)b * H + h;
        __syncthreads();  // the previous piece is done with sl, zl
        for (int x = threadIdx.x; x < R * R; x += blockDim.x) sl[x] = s[bh * R * R + x];
        if (threadIdx.x < R) zl[threadIdx.x] = z[bh * R + threadIdx.x];
        __syncthreads();
        float zreg[KQ];
#pragma unroll
        for (int t = 0; t < KQ; t++) zreg[t] = zl[feat(gq, t)];
        const int64_t col = h * R + 4 * gq;  // chunk c of the lane: features 16c + 4gq ..
        // the next tile's q rows stay raw until used, so their loads overlap this tile's
        // MFMAs; rows past the piece read its last row and are zeroed by a select
        v4f qn[KQ / 4];
        auto fetch = [&](int64_t rowt) {
            const int64_t row = rowt + li < r1 ? rowt + li : r1 - 1;
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) qn[c] = *reinterpret_cast<const v4f*>(q + row * W + col + 16 * c);
        };
        int64_t row0 = r0 + 16 * wave;
        if (row0 < r1) fetch(row0);
        for (; row0 < r1; row0 += 64) {
            float a[KQ];
            const bool ok = row0 + li < r1;
#pragma unroll
            for (int c = 0; c < KQ / 4; c++)
#pragma unroll
                for (int e = 0; e < 4; e++) a[4 * c + e] = ok ? phi(qn[c][e]) : 0.f;
            const int64_t nxt = row0 + 64;
            if (nxt < r1) fetch(nxt);
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < KQ; t++) d = fmaf(a[t], zreg[t], d);
            d += __shfl_xor(d, 16, 64);
            d += __shfl_xor(d, 32, 64);  // every lane li now holds the dot for row row0 + li
            v4f acc[TR];
#pragma unroll
            for (int j = 0; j < TR; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KQ; t++) {
                float sb[TR];
                lds_load_n<TR>(sl + feat(gq, t) * R + TR * li, sb);
#pragma unroll
                for (int j = 0; j < TR; j++)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], sb[j], acc[j], 0, 0, 0);
                if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // at most four steps' S loads live
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int rr = gq * 4 + q4;  // output row of this lane within the tile
                const float inv = 1.0f / (__shfl(d, rr, 64) + eps);
                const int64_t orow = row0 + rr;
                if (orow < r1) {
                    float o[TR];
#pragma unroll
                    for (int j = 0; j < TR; j++) o[j] = acc[j][q4] * inv;
                    store_n<TR>(g + orow * W + h * R + TR * li, o);
                }
            }
        }
    });
}

// Scalar path: one thread per output element.
__global__ void apply_scalar(Seg sg, int32_t H, int32_t R, float eps, const float* __restrict__ q,
                             const float* __restrict__ s, const float* __restrict__ z, float* __restrict__ g) {
    const int64_t W = (int64_t)H * R;
    for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < (int64_t)sg.n * W;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = x / W;
        const int h = (int)((x % W) / R), j = (int)(x % R);
        const int64_t bh = (int64_t)sg.graph_of(row) * H + h;
        const float* qr = q + row * W + h * R;
        float num = 0.f, d = 0.f;
        for (int c = 0; c < R; c++) {
            const float p = phi(qr[c]);
            num = fmaf(p, s[(bh * R + c) * R + j], num);
            d = fmaf(p, z[bh * R + c], d);
        }
        g[x] = num / (d + eps);
    }
}

// ======================================================================== backward
// Gradients of sum(G * dG) for the branch above, per graph and head, with S and z given:
//   num_i = phi(q_i)^T S, den_i = phi(q_i) . z + eps, G_i = num_i / den_i,
//   dnum_i = dG_i / den_i, dden_i = -(dG_i . G_i) / den_i,
//   dphi(q_i) = S dnum_i + z dden_i,   dS = sum_i phi(q_i) dnum_i^T,  dz = sum_i phi(q_i) dden_i,
//   dphi(k_j) = dS v_j + dz,           dv_j = dS^T phi(k_j),
// with the sums over the rows of the graph.  dq, dk, dv are accumulated (+=).

// Loads the R x R matrix m into LDS both as is and transposed, the columns of each copy
// permuted so that the TR entries a lane multiplies at MFMA position li of tiles 0..TR-1
// (columns li, 16 + li, ..) sit side by side: mr[c][TR*(j%16) + j/16] = m[c][j] and
// mt[j][TR*(c%16) + c/16] = m[c][j].
template <int TR>
__device__ __forceinline__ void stage_both(const float* __restrict__ m, float* mr, float* mt) {
    constexpr int R = TR * 16;
    for (int x = threadIdx.x; x < R * R; x += blockDim.x) {
        const float val = m[x];
        const int c = x / R, j = x % R;
        mr[c * R + TR * (j & 15) + (j >> 4)] = val;
        mt[j * R + TR * (c & 15) + (c >> 4)] = val;
    }
}

// ---- pass over the query rows, matrix-core path.  grid (tiles, H), 4 wavefronts per
// workgroup, all on head blockIdx.y; for each piece of the tile the wavefronts take its
// 16-row tiles in turn.  Per tile, with the lane layout feat (lane group gq holds features
// feat(gq, t) of the row li = lane%16):
//   1. dG . G, the one place num enters: with the forward's G given (HG), read beside dG;
//      otherwise num^T = S^T phi(Q)^T formed again: A = S read from LDS, B = phi(q) of the
//      lane's own row, so the output lands with row li in lane li and features
//      16jt + 4gq + q4 in group gq;
//   2. dphi(Q)^T = S dnum^T: A = S^T from LDS, B = the lane's own dnum;
//   3. dS += phi(Q)^T dnum: the tile's phi(q) and dnum go through LDS to put rows on the
//      contraction axis.
// The wavefronts' dS, dz sums are added in wavefront order and written as the piece's
// partial (same layout as the statistics), or as the graph's dS, dz for a short graph.
template <int TR, bool HG>
__global__ __launch_bounds__(256) void dq_mfma(Seg sg, int32_t H, float eps, const float* __restrict__ q,
                                               const float* __restrict__ s, const float* __restrict__ z,
                                               const float* __restrict__ dg, const float* __restrict__ gfw,
                                               float* __restrict__ dq,
                                               float* __restrict__ part, float* __restrict__ ds_out,
                                               float* __restrict__ dz_out) {
    constexpr int R = TR * 16, KQ = R / 4;
    __shared__ float sl[R * R], st[R * R];
    __shared__ float pq[4][16 * R], dn_l[4][16 * R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t tile = blockIdx.x;
    for_each_segment(sg, tile, [&](int32_t b, int64_t r0, int64_t r1, int slot) {
        const int64_t bh = (int64_t)b * H + h;
        __syncthreads();  // the previous piece is done with sl, st
        stage_both<TR>(s + bh * R * R, sl, st);
        float zreg[KQ];
#pragma unroll
        for (int t = 0; t < KQ; t++) zreg[t] = z[bh * R + feat(gq, t)];
        __syncthreads();

        v4f dsacc[TR][TR];
        float dzacc[KQ];
#pragma unroll
        for (int i = 0; i < TR; i++)
#pragma unroll
            for (int j = 0; j < TR; j++) dsacc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KQ; t++) dzacc[t] = 0.f;

        const int64_t ntile = (r1 - r0 + 15) / 16;
        const int64_t iters = (ntile + 3) / 4;
        for (int64_t it = 0; it < iters; it++) {
            const int64_t tl = it * 4 + wave;
            const int64_t row = r0 + tl * 16 + li;
            const bool valid = tl < ntile && row < r1;
            const int64_t off = row * W + h * R + 4 * gq;  // chunk c at off + 16c
            // q, dG (G with HG) and the dq being accumulated into are requested together, so
            // the dq values arrive during the products instead of after them; q itself is kept
            // only as phi(q) and a sign mask (phi'(q) is 1 where q > 0 and phi(q) elsewhere).
            float a[KQ], dgl[KQ], dqo[KQ], gv[HG ? KQ : 1];
            uint32_t pos = 0;
            if (valid) {
                float qr[KQ];
#pragma unroll
                for (int c = 0; c < KQ / 4; c++) {
                    const float4 t4 = *reinterpret_cast<const float4*>(q + off + 16 * c);
                    const float4 g4 = *reinterpret_cast<const float4*>(dg + off + 16 * c);
                    const float4 o4 = *reinterpret_cast<const float4*>(dq + off + 16 * c);
                    qr[4 * c + 0] = t4.x; qr[4 * c + 1] = t4.y; qr[4 * c + 2] = t4.z; qr[4 * c + 3] = t4.w;
                    dgl[4 * c + 0] = g4.x; dgl[4 * c + 1] = g4.y; dgl[4 * c + 2] = g4.z; dgl[4 * c + 3] = g4.w;
                    dqo[4 * c + 0] = o4.x; dqo[4 * c + 1] = o4.y; dqo[4 * c + 2] = o4.z; dqo[4 * c + 3] = o4.w;
                    if constexpr (HG) {
                        const float4 f4 = *reinterpret_cast<const float4*>(gfw + off + 16 * c);
                        gv[4 * c + 0] = f4.x; gv[4 * c + 1] = f4.y; gv[4 * c + 2] = f4.z; gv[4 * c + 3] = f4.w;
                    }
                }
#pragma unroll
                for (int t = 0; t < KQ; t++) {
                    a[t] = phi(qr[t]);
                    pos |= (qr[t] > 0.f ? 1u : 0u) << t;
                }
            } else {
#pragma unroll
                for (int t = 0; t < KQ; t++) a[t] = dgl[t] = dqo[t] = 0.f;
#pragma unroll
                for (int t = 0; t < (HG ? KQ : 1); t++) gv[t] = 0.f;
            }
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < KQ; t++) d = fmaf(a[t], zreg[t], d);
            d += __shfl_xor(d, 16, 64);
            d += __shfl_xor(d, 32, 64);
            const float inv = 1.0f / (d + eps);
            // 1. dG . G over the lane's features
            float dn[KQ];
            float dd = 0.f;
            if constexpr (HG) {
#pragma unroll
                for (int t = 0; t < KQ; t++) {
                    dd = fmaf(dgl[t], gv[t], dd);
                    dn[t] = dgl[t] * inv;
                }
            } else {
                v4f acc1[TR];
#pragma unroll
                for (int j = 0; j < TR; j++) acc1[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < KQ; t++) {
                    float sa[TR];
                    lds_load_n<TR>(sl + feat(gq, t) * R + TR * li, sa);
#pragma unroll
                    for (int j = 0; j < TR; j++)
                        acc1[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[j], a[t], acc1[j], 0, 0, 0);
                }
                // acc1[jt][q4] = num[row li][16jt + 4gq + q4], the lane's value t = 4jt + q4
#pragma unroll
                for (int j = 0; j < TR; j++)
#pragma unroll
                    for (int q4 = 0; q4 < 4; q4++) {
                        const int idx = 4 * j + q4;
                        dd = fmaf(dgl[idx], acc1[j][q4] * inv, dd);
                        dn[idx] = dgl[idx] * inv;
                    }
            }
            dd += __shfl_xor(dd, 16, 64);
            dd += __shfl_xor(dd, 32, 64);
            const float dden = -dd * inv;
            // 2. dphi(Q)^T
            v4f acc2[TR];
#pragma unroll
            for (int j = 0; j < TR; j++) acc2[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KQ; t++) {
                float sa[TR];
                lds_load_n<TR>(st + feat(gq, t) * R + TR * li, sa);
#pragma unroll
                for (int c = 0; c < TR; c++)
                    acc2[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[c], dn[t], acc2[c], 0, 0, 0);
            }
            // acc2[ct][q4] = (S dnum)[row li][16ct + 4gq + q4], the lane's value t = 4ct + q4
            if (valid) {
#pragma unroll
                for (int c = 0; c < KQ / 4; c++) {
                    float u[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int idx = 4 * c + e;
                        const float gv = acc2[c][e] + zreg[idx] * dden;
                        u[e] = dqo[idx] + gv * ((pos >> idx) & 1u ? 1.f : a[idx]);
                    }
                    *reinterpret_cast<float4*>(dq + off + 16 * c) = make_float4(u[0], u[1], u[2], u[3]);
                }
            }
#pragma unroll
            for (int t = 0; t < KQ; t++) dzacc[t] = fmaf(a[t], dden, dzacc[t]);
            // 3. dS += phi(Q)^T dnum, rows moved onto the contraction axis through LDS
            float* pw = pq[wave];
            float* dw = dn_l[wave];
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
                *reinterpret_cast<float4*>(pw + li * R + 16 * c + 4 * gq) =
                    make_float4(a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]);
                *reinterpret_cast<float4*>(dw + li * R + 16 * c + 4 * gq) =
                    make_float4(dn[4 * c], dn[4 * c + 1], dn[4 * c + 2], dn[4 * c + 3]);
            }
            wave_lds_sync();  // pq[wave], dn_l[wave] belong to this wavefront alone
#pragma unroll
            for (int u = 0; u < 4; u++) {
                float pa[TR], pb[TR];
                lds_load_n<TR>(pw + (4 * u + gq) * R + TR * li, pa);
                lds_load_n<TR>(dw + (4 * u + gq) * R + TR * li, pb);
#pragma unroll
                for (int i = 0; i < TR; i++)
#pragma unroll
                    for (int j = 0; j < TR; j++)
                        dsacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[i], pb[j], dsacc[i][j], 0, 0, 0);
            }
            wave_lds_sync();  // read before the next tile overwrites them
        }
        __syncthreads();  // every wavefront is done reading sl, st before they take the sums
        // dz over the 16 rows of the lane group
#pragma unroll
        for (int t = 0; t < KQ; t++) {
            float v = dzacc[t];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            dzacc[t] = v;
        }
        // wavefronts add into sl (R*R) + st (first R) in wavefront order; each element has
        // one owner lane
        float* buf = sl;
        float* zbuf = st;
        for (int w = 0; w < 4; w++) {
            if (wave == w) {
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
#pragma unroll
                    for (int i = 0; i < TR; i++)
#pragma unroll
                        for (int j = 0; j < TR; j++) {
                            const int e = (TR * (gq * 4 + q4) + i) * R + TR * li + j;
                            buf[e] = (w == 0 ? 0.f : buf[e]) + dsacc[i][j][q4];
                        }
                if (li == 0) {
#pragma unroll
                    for (int t = 0; t < KQ; t++) zbuf[feat(gq, t)] = (w == 0 ? 0.f : zbuf[feat(gq, t)]) + dzacc[t];
                }
            }
            __syncthreads();
        }
        if (slot >= 0) {
            float* out = part + ((tile * 2 + slot) * H + h) * (R * R + R);
            for (int x = threadIdx.x; x < R * R + R; x += blockDim.x) out[x] = x < R * R ? buf[x] : zbuf[x - R * R];
        } else {
            for (int x = threadIdx.x; x < R * R + R; x += blockDim.x) {
                if (x < R * R)
                    ds_out[bh * R * R + x] = buf[x];
                else
                    dz_out[bh * R + x - R * R] = zbuf[x - R * R];
            }
        }
    });
}

// ---- pass over the key rows, matrix-core path.  grid (tiles, H), 4 wavefronts per
// workgroup on head blockIdx.y.  For each piece the graph's dS and dS^T sit in LDS and the
// wavefronts take the piece's 16-row tiles in turn:
//   dphi(K)^T = dS V^T: A = dS^T rows, B = the lane's own v;
//   dV^T = dS^T phi(K)^T: A = dS rows, B = the lane's own phi(k).
// The next tile's k and v are loaded before the current tile's products, the dk, dv it adds
// to after them (holding them through the products cost registers and measured 3.5% slower);
// registers are held to two wavefronts per SIMD so that one wavefront's loads overlap the
// other's products.
template <int TR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dkv_mfma(
    Seg sg, int32_t H, const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ ds,
    const float* __restrict__ dz, float* __restrict__ dk, float* __restrict__ dv) {
    constexpr int R = TR * 16, KQ = R / 4;
    __shared__ float sl[R * R], st[R * R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    for_each_segment(sg, blockIdx.x, [&](int32_t b, int64_t r0, int64_t r1, int) {
        const int64_t bh = (int64_t)b * H + h;
        __syncthreads();
        stage_both<TR>(ds + bh * R * R, sl, st);
        float zreg[KQ];
#pragma unroll
        for (int t = 0; t < KQ; t++) zreg[t] = dz[bh * R + feat(gq, t)];
        __syncthreads();
        // the next tile's k and v, loaded during the current tile's products
        v4f kx[KQ / 4], vx[KQ / 4];
        auto fetch = [&](int64_t row0) {
            const int64_t row = row0 + li;
            const int64_t off = row * W + h * R + 4 * gq;  // chunk c at off + 16c
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
                kx[c] = vx[c] = v4f{0.f, 0.f, 0.f, 0.f};
                if (row < r1) {
                    kx[c] = *reinterpret_cast<const v4f*>(k + off + 16 * c);
                    vx[c] = *reinterpret_cast<const v4f*>(v + off + 16 * c);
                }
            }
        };
        int64_t row0 = r0 + wave * 16;
        if (row0 < r1) fetch(row0);
        for (; row0 < r1; row0 += 64) {
            const int64_t row = row0 + li;
            const bool valid = row < r1;
            const int64_t off = row * W + h * R + 4 * gq;  // chunk c at off + 16c
            float pk[KQ], vv[KQ];
            uint32_t pos = 0;              // bit t: k feature t > 0, where dphi = 1
#pragma unroll
            for (int c = 0; c < KQ / 4; c++) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float x = kx[c][e];
                    pk[4 * c + e] = valid ? phi(x) : 0.f;
                    pos |= (x > 0.f ? 1u : 0u) << (4 * c + e);
                    vv[4 * c + e] = vx[c][e];
                }
            }
            if (row0 + 64 < r1) fetch(row0 + 64);
            v4f ak[TR], av[TR];
#pragma unroll
            for (int j = 0; j < TR; j++) ak[j] = av[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KQ; t++) {
                float sa[TR], sb[TR];
                lds_load_n<TR>(st + feat(gq, t) * R + TR * li, sa);
                lds_load_n<TR>(sl + feat(gq, t) * R + TR * li, sb);
#pragma unroll
                for (int j = 0; j < TR; j++) {
                    ak[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[j], vv[t], ak[j], 0, 0, 0);
                    av[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sb[j], pk[t], av[j], 0, 0, 0);
                }
                if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // at most four steps' dS loads live
            }
            // ak[ct][q4] = (dS v)[row li][16ct + 4gq + q4], the lane's value t = 4ct + q4; av
            // likewise for dS^T phi(k)
            if (valid) {
                v4f odk[KQ / 4], odv[KQ / 4];
#pragma unroll
                for (int c = 0; c < KQ / 4; c++) {
                    odk[c] = *reinterpret_cast<const v4f*>(dk + off + 16 * c);
                    odv[c] = *reinterpret_cast<const v4f*>(dv + off + 16 * c);
                }
#pragma unroll
                for (int c = 0; c < KQ / 4; c++) {
                    v4f ok, ov;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int idx = 4 * c + e;
                        const float dp = (pos >> idx) & 1u ? 1.f : pk[idx];  // dphi
                        ok[e] = odk[c][e] + (ak[c][e] + zreg[idx]) * dp;
                        ov[e] = odv[c][e] + av[c][e];
                    }
                    *reinterpret_cast<v4f*>(dk + off + 16 * c) = ok;
                    *reinterpret_cast<v4f*>(dv + off + 16 * c) = ov;
                }
            }
        }
    });
}

// ---- scalar paths (any r <= 64): one wavefront per row and head, lane c <-> feature c.
// Query pass: grid (tiles, H), 4 wavefronts per workgroup taking the piece's rows in turn;
// the piece's dS, dz as above.
__global__ __launch_bounds__(256) void dq_scalar(Seg sg, int32_t H, int32_t R, float eps, const float* __restrict__ q,
                                                 const float* __restrict__ s, const float* __restrict__ z,
                                                 const float* __restrict__ dg, const float* __restrict__ gfw,
                                                 float* __restrict__ dq,
                                                 float* __restrict__ part, float* __restrict__ ds_out,
                                                 float* __restrict__ dz_out) {
    __shared__ float buf[64 * 64 + 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const int64_t tile = blockIdx.x;
    const bool on = lane < R;
    for_each_segment(sg, tile, [&](int32_t b, int64_t r0, int64_t r1, int slot) {
        const int64_t bh = (int64_t)b * H + h;
        const float* sh = s + bh * R * R;
        const float zc = on ? z[bh * R + lane] : 0.f;
        float acc[64];  // acc[c] = dS[c][lane]
#pragma unroll
        for (int c = 0; c < 64; c++) acc[c] = 0.f;
        float dzacc = 0.f;
        for (int64_t row = r0 + wave; row < r1; row += 4) {
            const int64_t off = row * W + h * R + lane;
            const float qc = on ? q[off] : 0.f;
            const float pc = on ? phi(qc) : 0.f;
            float d = pc * zc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) d += __shfl_xor(d, o, 64);
            const float inv = 1.0f / (d + eps);
            float gj;  // G of this feature: the forward's, or num / den formed again
            if (gfw) {
                gj = on ? gfw[off] : 0.f;
            } else {
                float num = 0.f;
                for (int c = 0; c < R; c++) num = fmaf(__shfl(pc, c, 64), on ? sh[c * R + lane] : 0.f, num);
                gj = num * inv;
            }
            const float dgj = on ? dg[off] : 0.f;
            float dd = dgj * gj;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) dd += __shfl_xor(dd, o, 64);
            const float dden = -dd * inv;
            const float dnj = dgj * inv;
            float dp = 0.f;
            for (int j = 0; j < R; j++) dp = fmaf(on ? sh[lane * R + j] : 0.f, __shfl(dnj, j, 64), dp);
            if (on) dq[off] += (dp + zc * dden) * dphi(qc, pc);
#pragma unroll
            for (int c = 0; c < 64; c++)
                if (c < R) acc[c] = fmaf(__shfl(pc, c, 64), dnj, acc[c]);
            dzacc = fmaf(pc, dden, dzacc);
        }
        __syncthreads();  // the previous piece's copy-out is done with buf
        for (int w = 0; w < 4; w++) {
            if (wave == w && on) {
#pragma unroll
                for (int c = 0; c < 64; c++)
                    if (c < R) buf[c * R + lane] = (w == 0 ? 0.f : buf[c * R + lane]) + acc[c];
                buf[R * R + lane] = (w == 0 ? 0.f : buf[R * R + lane]) + dzacc;
            }
            __syncthreads();
        }
        if (slot >= 0) {
            float* out = part + ((tile * 2 + slot) * H + h) * (R * R + R);
            for (int x = threadIdx.x; x < R * R + R; x += blockDim.x) out[x] = buf[x];
        } else {
            for (int x = threadIdx.x; x < R * R + R; x += blockDim.x) {
                if (x < R * R)
                    ds_out[bh * R * R + x] = buf[x];
                else
                    dz_out[bh * R + x - R * R] = buf[x];
            }
        }
    });
}

// Key pass: one wavefront per row and head (grid-strided rows), dS of the row's graph.
__global__ __launch_bounds__(256) void dkv_scalar(Seg sg, int32_t H, int32_t R, const float* __restrict__ k,
                                                  const float* __restrict__ v, const float* __restrict__ ds,
                                                  const float* __restrict__ dz, float* __restrict__ dk,
                                                  float* __restrict__ dv) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y;
    const int64_t W = (int64_t)H * R;
    const bool on = lane < R;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < sg.n; row += (int64_t)gridDim.x * 4) {
        const int64_t bh = (int64_t)sg.graph_of(row) * H + h;
        const float* sh = ds + bh * R * R;
        const float zc = on ? dz[bh * R + lane] : 0.f;
        const int64_t off = row * W + h * R + lane;
        const float kc = on ? k[off] : 0.f, vc = on ? v[off] : 0.f;
        const float pc = on ? phi(kc) : 0.f;
        float a = 0.f, b = 0.f;
        for (int j = 0; j < R; j++) a = fmaf(on ? sh[lane * R + j] : 0.f, __shfl(vc, j, 64), a);
        for (int c = 0; c < R; c++) b = fmaf(on ? sh[c * R + lane] : 0.f, __shfl(pc, c, 64), b);
        if (on) {
            dk[off] += (a + zc) * dphi(kc, pc);
            dv[off] += b;
        }
    }
}

// ---------------------------------------------------------------- host side

// Rows per tile: a multiple of 16, at least 256, and large enough for at most 1024 / heads
// tiles.  Every kernel here runs a workgroup per (tile, head), and each workgroup stages S
// (and its transpose) and writes a partial of r x r + r sums besides its rows: about 1024
// workgroups fill the chip, and longer tiles spread that fixed cost over more rows (at 4
// heads of 64 and 2^18 rows, 256 tiles against 1024: forward 297 -> 248 us, backward
// 780 -> 703 us; 128 tiles, 512 workgroups, left CUs idle: forward 404 us).
int32_t tile_rows(int32_t n, int32_t heads) {
    const int64_t cap = heads < 1024 ? 1024 / heads : 1;
    int64_t per = ((int64_t)n + cap - 1) / cap;
    per = (per + 15) / 16 * 16;
    return (int32_t)(per < 256 ? 256 : per);
}

int64_t tile_count(int32_t n, int32_t rs) { return n > 0 ? ((int64_t)n + rs - 1) / rs : 0; }

struct GlWs {
    float* part;    // [2 * tiles][H][R*R + R] pieces of long graphs
    float* s;       // [batch][H][R*R]  S (forward) or dS (backward)
    float* z;       // [batch][H][R]    z or dz
    int4* list;      // [tiles] long graphs (first tile, graph, rows)
    int32_t* count;  // number of long graphs
    size_t bytes;
};

GlWs carve_gl(void* ws, int32_t n, int32_t batch, int32_t H, int32_t R) {
    const int64_t tiles = tile_count(n, tile_rows(n, H));
    Carver c(ws);
    GlWs w;
    w.part = c.take<float>((size_t)(tiles > 0 ? 2 * tiles : 1) * H * (R * R + R));
    w.s = c.take<float>((size_t)batch * H * R * R);
    w.z = c.take<float>((size_t)batch * H * R);
    w.list = c.take<int4>((size_t)(tiles > 0 ? tiles : 1));
    w.count = c.take<int32_t>(1);
    w.bytes = c.bytes();
    return w;
}

void launch_list_and_reduce(const Seg& sg, int32_t H, int32_t R, const GlWs& w, float* s, float* z, hipStream_t st) {
    const int64_t tiles = tile_count(sg.n, sg.rs);
    list_long<<<1, 1024, 0, st>>>(sg, tiles, w.list, w.count);
    const int64_t longest = tiles < sg.batch ? tiles : sg.batch;  // long graphs: at most one per tile
    const int64_t tot = (int64_t)H * (R * R + R);
    const unsigned gx = (unsigned)((tot + 63) / 64);
    // one graph: its (up to 1024) tiles over 16 wavefronts per output; a batch: 4 wavefronts
    // and more graphs at once (a fixed choice per shape, so the order of the sums is too)
    if (sg.batch == 1) {
        seg_reduce<16><<<dim3(gx, 1), 1024, 0, st>>>(sg, H, R, w.list, w.count, w.part, s, z);
    } else {
        const unsigned gy = (unsigned)(longest < 256 ? (longest > 0 ? longest : 1) : 256);
        seg_reduce<4><<<dim3(gx, gy), 256, 0, st>>>(sg, H, R, w.list, w.count, w.part, s, z);
    }
}

bool mfma_ok(int32_t r) { return r % 16 == 0 && r <= 64; }

int gl_fwd(const Seg& sg, int32_t heads, int32_t r, const float* q, const float* k, const float* v, float eps,
           float* s_out, float* z_out, float* g_out, void* ws, size_t ws_bytes, hipStream_t st) {
    const GlWs need = carve_gl(nullptr, sg.n, sg.batch, heads, r);
    if (ws_bytes < need.bytes || !ws) return GGA_EWORKSPACE;
    const GlWs w = carve_gl(ws, sg.n, sg.batch, heads, r);
    float* s = s_out ? s_out : w.s;
    float* z = z_out ? z_out : w.z;
    // graphs with no rows keep S = 0, z = 0
    if (sg.node_ptr || sg.n == 0) {
        fill_f32(s, (int64_t)sg.batch * heads * r * r, 0.f, st);
        fill_f32(z, (int64_t)sg.batch * heads * r, 0.f, st);
    }
    if (sg.n == 0) return launch_status();
    const int64_t tiles = tile_count(sg.n, sg.rs);
    const bool mfma = mfma_ok(r) && aligned16(q) && aligned16(k) && aligned16(v) && aligned16(g_out) &&
                      aligned16(s) && aligned16(z);
    const int wpb = heads < 8 ? heads : 8;  // wavefronts (heads) per workgroup
    if (mfma) {
        const unsigned grid = (unsigned)tiles, threads = 64u * wpb;
        switch (r / 16) {
            case 1: stats_mfma<1><<<grid, threads, 0, st>>>(sg, heads, k, v, w.part, s, z); break;
            case 2: stats_mfma<2><<<grid, threads, 0, st>>>(sg, heads, k, v, w.part, s, z); break;
            case 3: stats_mfma<3><<<grid, threads, 0, st>>>(sg, heads, k, v, w.part, s, z); break;
            default: stats_mfma<4><<<grid, threads, 0, st>>>(sg, heads, k, v, w.part, s, z); break;
        }
    } else {
        stats_scalar<<<dim3((unsigned)tiles, (unsigned)heads), 256, 0, st>>>(sg, heads, r, k, v, w.part, s, z);
    }
    launch_list_and_reduce(sg, heads, r, w, s, z, st);
    if (mfma) {
        const dim3 ga((unsigned)tiles, (unsigned)heads);
        switch (r / 16) {
            case 1: apply_mfma<1><<<ga, 256, 0, st>>>(sg, heads, eps, q, s, z, g_out); break;
            case 2: apply_mfma<2><<<ga, 256, 0, st>>>(sg, heads, eps, q, s, z, g_out); break;
            case 3: apply_mfma<3><<<ga, 256, 0, st>>>(sg, heads, eps, q, s, z, g_out); break;
            default: apply_mfma<4><<<ga, 256, 0, st>>>(sg, heads, eps, q, s, z, g_out); break;
        }
    } else {
        int64_t blocks = ((int64_t)sg.n * heads * r + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        apply_scalar<<<(unsigned)blocks, 256, 0, st>>>(sg, heads, r, eps, q, s, z, g_out);
    }
    return launch_status();
}

int gl_bwd(const Seg& sg, int32_t heads, int32_t r, const float* q, const float* k, const float* v, float eps,
           const float* s_in, const float* z_in, const float* d_g, const float* g_fw, float* d_q, float* d_k,
           float* d_v, void* ws, size_t ws_bytes, hipStream_t st) {
    const GlWs need = carve_gl(nullptr, sg.n, sg.batch, heads, r);
    if (ws_bytes < need.bytes || !ws) return GGA_EWORKSPACE;
    if (sg.n == 0) return GGA_OK;
    const GlWs w = carve_gl(ws, sg.n, sg.batch, heads, r);
    if (sg.node_ptr) {  // graphs with no rows: dS = 0, dz = 0 (never read, kept defined)
        fill_f32(w.s, (int64_t)sg.batch * heads * r * r, 0.f, st);
        fill_f32(w.z, (int64_t)sg.batch * heads * r, 0.f, st);
    }
    const int64_t tiles = tile_count(sg.n, sg.rs);
    const bool mfma = mfma_ok(r) && aligned16(q) && aligned16(k) && aligned16(v) && aligned16(d_g) &&
                      aligned16(d_q) && aligned16(d_k) && aligned16(d_v) && aligned16(g_fw);
    const dim3 ga((unsigned)tiles, (unsigned)heads);
    if (mfma) {
#define GGA_DQ(TR)                                                                                              \
    if (g_fw)                                                                                                   \
        dq_mfma<TR, true><<<ga, 256, 0, st>>>(sg, heads, eps, q, s_in, z_in, d_g, g_fw, d_q, w.part, w.s, w.z);  \
    else                                                                                                        \
        dq_mfma<TR, false><<<ga, 256, 0, st>>>(sg, heads, eps, q, s_in, z_in, d_g, g_fw, d_q, w.part, w.s, w.z)
        switch (r / 16) {
            case 1: GGA_DQ(1); break;
            case 2: GGA_DQ(2); break;
            case 3: GGA_DQ(3); break;
            default: GGA_DQ(4); break;
        }
#undef GGA_DQ
    } else {
        dq_scalar<<<ga, 256, 0, st>>>(sg, heads, r, eps, q, s_in, z_in, d_g, g_fw, d_q, w.part, w.s, w.z);
    }
    launch_list_and_reduce(sg, heads, r, w, w.s, w.z, st);
    if (mfma) {
        switch (r / 16) {
            case 1: dkv_mfma<1><<<ga, 256, 0, st>>>(sg, heads, k, v, w.s, w.z, d_k, d_v); break;
            case 2: dkv_mfma<2><<<ga, 256, 0, st>>>(sg, heads, k, v, w.s, w.z, d_k, d_v); break;
            case 3: dkv_mfma<3><<<ga, 256, 0, st>>>(sg, heads, k, v, w.s, w.z, d_k, d_v); break;
            default: dkv_mfma<4><<<ga, 256, 0, st>>>(sg, heads, k, v, w.s, w.z, d_k, d_v); break;
        }
    } else {
        int64_t blocks = ((int64_t)sg.n + 3) / 4;
        if (blocks > 4096) blocks = 4096;
        dkv_scalar<<<dim3((unsigned)blocks, (unsigned)heads), 256, 0, st>>>(sg, heads, r, k, v, w.s, w.z, d_k, d_v);
    }
    return launch_status();
}

Seg one_graph(int32_t n, int32_t heads) { return Seg{nullptr, 1, n, tile_rows(n, heads)}; }

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" size_t gga_global_linear_workspace(int32_t n, int32_t heads, int32_t r) {
    if (n < 0 || heads < 1 || r < 1) return 0;
    return carve_gl(nullptr, n, 1, heads, r).bytes;
}

extern "C" int gga_global_linear_fwd(int32_t n, int32_t heads, int32_t r, const float* q, const float* k,
                                     const float* v, float eps, float* s_out, float* z_out, float* g_out, void* ws,
                                     size_t ws_bytes, void* stream) {
    if (n < 0 || heads < 1 || r < 1) return GGA_EINVAL;
    if (r > 1024) return GGA_EUNSUPPORTED;
    if (heads > 65535) return GGA_ERANGE;
    if (n > 0 && (!q || !k || !v || !g_out)) return GGA_EINVAL;
    return gl_fwd(one_graph(n, heads), heads, r, q, k, v, eps, s_out, z_out, g_out, ws, ws_bytes, as_stream(stream));
}

extern "C" size_t gga_global_linear_bwd_workspace(int32_t n, int32_t heads, int32_t r) {
    if (n < 0 || heads < 1 || r < 1) return 0;
    return carve_gl(nullptr, n, 1, heads, r).bytes;
}

extern "C" int gga_global_linear_bwd(int32_t n, int32_t heads, int32_t r, const float* q, const float* k,
                                     const float* v, float eps, const float* s_in, const float* z_in, const float* d_g,
                                     const float* g_fw, float* d_q, float* d_k, float* d_v, void* ws, size_t ws_bytes,
                                     void* stream) {
    if (n < 0 || heads < 1 || r < 1) return GGA_EINVAL;
    if (r > 64) return GGA_EUNSUPPORTED;
    if (heads > 65535) return GGA_ERANGE;
    if (n == 0) return GGA_OK;
    if (!q || !k || !v || !s_in || !z_in || !d_g || !d_q || !d_k || !d_v) return GGA_EINVAL;
    return gl_bwd(one_graph(n, heads), heads, r, q, k, v, eps, s_in, z_in, d_g, g_fw, d_q, d_k, d_v, ws, ws_bytes,
                  as_stream(stream));
}

extern "C" size_t gga_global_linear_batch_workspace(int32_t n, int32_t batch, int32_t heads, int32_t r) {
    if (n < 0 || batch < 1 || heads < 1 || r < 1) return 0;
    return carve_gl(nullptr, n, batch, heads, r).bytes;
}

extern "C" int gga_global_linear_batch_fwd(int32_t n, int32_t batch, const int32_t* node_ptr, int32_t heads,
                                           int32_t r, const float* q, const float* k, const float* v, float eps,
                                           float* s_out, float* z_out, float* g_out, void* ws, size_t ws_bytes,
                                           void* stream) {
    if (n < 0 || batch < 1 || heads < 1 || r < 1) return GGA_EINVAL;
    if (r > 1024) return GGA_EUNSUPPORTED;
    if (heads > 65535) return GGA_ERANGE;
    if (!node_ptr || (n > 0 && (!q || !k || !v || !g_out))) return GGA_EINVAL;
    const Seg sg{node_ptr, batch, n, tile_rows(n, heads)};
    return gl_fwd(sg, heads, r, q, k, v, eps, s_out, z_out, g_out, ws, ws_bytes, as_stream(stream));
}

extern "C" int gga_global_linear_batch_bwd(int32_t n, int32_t batch, const int32_t* node_ptr, int32_t heads,
                                           int32_t r, const float* q, const float* k, const float* v, float eps,
                                           const float* s_in, const float* z_in, const float* d_g,
                                           const float* g_fw, float* d_q, float* d_k, float* d_v, void* ws,
                                           size_t ws_bytes, void* stream) {
    if (n < 0 || batch < 1 || heads < 1 || r < 1) return GGA_EINVAL;
    if (r > 64) return GGA_EUNSUPPORTED;
    if (heads > 65535) return GGA_ERANGE;
    if (n == 0) return GGA_OK;
    if (!node_ptr || !q || !k || !v || !s_in || !z_in || !d_g || !d_q || !d_k || !d_v) return GGA_EINVAL;
    const Seg sg{node_ptr, batch, n, tile_rows(n, heads)};
    return gl_bwd(sg, heads, r, q, k, v, eps, s_in, z_in, d_g, g_fw, d_q, d_k, d_v, ws, ws_bytes,
                  as_stream(stream));
}
