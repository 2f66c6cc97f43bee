// Dense fp32 product on the matrix cores (v_mfma_f32_16x16x4_f32): c = op(a) op(b) (+ bias),
// or c += op(a) op(b).
//
// Kernels by shape:
// - n > 64: gemm_f32_big, 128 x 128 tiles of four wavefronts, each operand staged in LDS in
//   the layout its memory order gives (see its comment);
// - n <= 64: gemm_f32_mfma<64>, 128 x 64 tiles of eight wavefronts, both operands staged as
//   [row][k];
// - k, n <= 32: gemm_rows (a thread per output row); k, n <= 64: gemm_narrow;
// - a transposed a with few outputs over a long k: gemm_outer (m, n <= 16, one MFMA tile)
//   or gemm_small_out (m, n <= 32).
// When the output has few tiles and k is long, k is split into a fixed number of ranges whose
// partial products are added in a fixed order by a second kernel, so results do not depend on
// scheduling.
#include "common.hpp"

namespace gga {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, KT = 16;

constexpr int kMaxSegs = 4;

struct GemmArgs {
    const float* a;
    const float* b;
    const float* bias;
    float* c;
    int32_t M, K, N, lda, ldb;
    int32_t trans_a, trans_b;
    int32_t kchunk;  // K range per split
    int32_t accumulate;  // add into c instead of overwriting it
    // Segmented operands (plain a and plain b only; seg_len a multiple of the 128-wide tile
    // for column segments, of the 32-deep stage for k segments).  nseg > 1: the columns
    // [s seg_len, (s+1) seg_len) of op(b) and c are the matrices seg_b[s] [K, seg_len] and
    // seg_c[s] [M, seg_len].  kseg > 1: the k range [s seg_len, (s+1) seg_len) of a and b is
    // seg_a[s] [M, seg_len] and seg_b[s] [seg_len, N], added in segment order.
    int32_t nseg, kseg, seg_len;
    const float* seg_a[kMaxSegs];
    const float* seg_b[kMaxSegs];
    float* seg_c[kMaxSegs];
    // gate_out != null: the workgroups of column tile 0 also write gate_out[i] = a[i,:] . gate_w
    // + gate_b for their rows, from the a values they load anyway (plain a only).
    const float* gate_w;
    float* gate_out;
    float gate_b;
    // r1_row != null (gemm_f32_seg_k only): c also gets the outer product r1_row r1_col^T
    // (r1_row [M], r1_col [N]), added in the epilogue with the accumulation.
    const float* r1_row;
    const float* r1_col;
};

// Loads 4 consecutive floats of a row starting at column c0, zero beyond `lim` columns.
__device__ __forceinline__ float4 load4(const float* row, int64_t c0, int64_t lim, bool vec_ok) {
    if (vec_ok && c0 + 3 < lim) return *reinterpret_cast<const float4*>(row + c0);
    float4 r;
    r.x = c0 + 0 < lim ? row[c0 + 0] : 0.f;
    r.y = c0 + 1 < lim ? row[c0 + 1] : 0.f;
    r.z = c0 + 2 < lim ? row[c0 + 2] : 0.f;
    r.w = c0 + 3 < lim ? row[c0 + 3] : 0.f;
    return r;
}

constexpr int kGemmThreads = 512;  // 8 wavefronts: 2 along m x 4 along n

// Number of float4 a thread moves for an operand tile of width TW (along m or n) x KT.
template <int TW>
constexpr int tile_q() { return (TW * KT / 4 + kGemmThreads - 1) / kGemmThreads; }

// One operand tile (TW along m or n, KT along k) into registers.
// `kmajor_src`: the operand is stored with k as its row index (a transposed / b plain).
template <int TW>
__device__ __forceinline__ void fetch_tile(const float* src, int ld, bool kmajor_src, int64_t o0, int64_t olim,
                                           int64_t k0, int64_t klim, bool vec_ok, float4 (&r)[tile_q<TW>()]) {
#pragma unroll
    for (int q = 0; q < tile_q<TW>(); q++) {
        const int f = threadIdx.x + kGemmThreads * q;
        r[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (f >= TW * KT / 4) continue;
        if (kmajor_src) {
            // k fastest across threads: the transposing LDS store then hits consecutive banks
            const int kr = f % KT, c4 = f / KT;
            const int64_t k = k0 + kr;
            if (k < klim) r[q] = load4(src + k * ld, o0 + c4 * 4, olim, vec_ok);
        } else {
            const int orow = f / (KT / 4), c4 = f % (KT / 4);
            const int64_t o = o0 + orow;
            if (o < olim) r[q] = load4(src + o * ld, k0 + c4 * 4, klim, vec_ok);
        }
    }
}

// LDS holds each operand tile as [row][k] (rows along m or n), KT + 4 floats per row.
constexpr int LDS_ROW = KT + 4;

// A k-major source is transposed on its way into LDS; otherwise rows are copied as
// 16-byte vectors.
template <int TW>
__device__ __forceinline__ void stash_tile(float* lds, bool kmajor_src, const float4 (&r)[tile_q<TW>()]) {
#pragma unroll
    for (int q = 0; q < tile_q<TW>(); q++) {
        const int f = threadIdx.x + kGemmThreads * q;
        if (f >= TW * KT / 4) continue;
        if (kmajor_src) {
            const int kr = f % KT, c4 = f / KT;
            lds[(c4 * 4 + 0) * LDS_ROW + kr] = r[q].x;
            lds[(c4 * 4 + 1) * LDS_ROW + kr] = r[q].y;
            lds[(c4 * 4 + 2) * LDS_ROW + kr] = r[q].z;
            lds[(c4 * 4 + 3) * LDS_ROW + kr] = r[q].w;
        } else {
            const int orow = f / (KT / 4), c4 = f % (KT / 4);
            *reinterpret_cast<float4*>(lds + orow * LDS_ROW + c4 * 4) = r[q];
        }
    }
}

// MFMAs of one KT-deep LDS tile into a wavefront's 64 x (BN/4) accumulators.  The
// contraction index is permuted inside the tile: MFMA step t takes, in the k slot of lane
// group g = lane/16, the element k = 4g + t, so each lane's operands for the four steps are
// four consecutive k of one row -- one 16-byte LDS read per operand tile.
template <int BN>
__device__ __forceinline__ void mfma_tile(const float* as, const float* bs, int wm, int wn, int lane,
                                          v4f (&acc)[4][BN / 64]) {
    constexpr int TJ = BN / 64;
    const int kq = (lane >> 4) * 4;
    float4 af[4], bf[TJ];
#pragma unroll
    for (int i = 0; i < 4; i++)
        af[i] = *reinterpret_cast<const float4*>(as + (wm * 64 + i * 16 + (lane & 15)) * LDS_ROW + kq);
#pragma unroll
    for (int j = 0; j < TJ; j++)
        bf[j] = *reinterpret_cast<const float4*>(bs + (wn * (BN / 4) + j * 16 + (lane & 15)) * LDS_ROW + kq);
#pragma unroll
    for (int st = 0; st < 4; st++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float av = st == 0 ? af[i].x : st == 1 ? af[i].y : st == 2 ? af[i].z : af[i].w;
#pragma unroll
            for (int j = 0; j < TJ; j++) {
                const float bv = st == 0 ? bf[j].x : st == 1 ? bf[j].y : st == 2 ? bf[j].z : bf[j].w;
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[i][j], 0, 0, 0);
            }
        }
    }
}

// grid: (ceil(N/BN), ceil(M/BM), splits).  With splits > 1, c points at the partial buffer
// [splits][M][N] and bias is ignored.  Wavefront w owns rows (w/4)*64 .. +64 and columns
// (w%4)*BN/4 .. +BN/4 of the workgroup tile.
template <int BN>
__global__ __launch_bounds__(kGemmThreads) void gemm_f32_mfma(GemmArgs g) {
    constexpr int TJ = BN / 64;
    __shared__ float As[2][BM * LDS_ROW];
    __shared__ float Bs[2][BN * LDS_ROW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    // tiles in (split, row tile, column tile) order, each XCD taking a contiguous range, so
    // the column tiles of one row tile share an L2
    const uint32_t gxy = gridDim.x * gridDim.y;
    const uint32_t t = xcd_order(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gxy * gridDim.z);
    const uint32_t bz = t / gxy, by = (t % gxy) / gridDim.x, bx = t % gridDim.x;
    const int64_t m0 = (int64_t)by * BM, n0 = (int64_t)bx * BN;
    const int64_t kb = (int64_t)bz * g.kchunk;
    const int64_t ke = kb + g.kchunk < g.K ? kb + g.kchunk : g.K;
    const bool a_km = g.trans_a != 0;   // a stored [K][M]
    const bool b_km = g.trans_b == 0;   // b stored [K][N]
    const bool a_vec = (g.lda % 4) == 0 && (reinterpret_cast<uintptr_t>(g.a) & 15) == 0;
    const bool b_vec = (g.ldb % 4) == 0 && (reinterpret_cast<uintptr_t>(g.b) & 15) == 0;

    v4f acc[4][TJ];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)((ke - kb + KT - 1) / KT);
    float4 ra[tile_q<BM>()], rb[tile_q<BN>()];
    if (nk > 0) {
        fetch_tile<BM>(g.a, g.lda, a_km, m0, g.M, kb, ke, a_vec, ra);
        fetch_tile<BN>(g.b, g.ldb, b_km, n0, g.N, kb, ke, b_vec, rb);
        stash_tile<BM>(As[0], a_km, ra);
        stash_tile<BN>(Bs[0], b_km, rb);
    }
    __syncthreads();
    for (int t = 0; t < nk; t++) {
        const int cur = t & 1;
        if (t + 1 < nk) {
            const int64_t k0 = kb + (int64_t)(t + 1) * KT;
            fetch_tile<BM>(g.a, g.lda, a_km, m0, g.M, k0, ke, a_vec, ra);
            fetch_tile<BN>(g.b, g.ldb, b_km, n0, g.N, k0, ke, b_vec, rb);
        }
        mfma_tile<BN>(As[cur], Bs[cur], wm, wn, lane, acc);
        if (t + 1 < nk) {
            stash_tile<BM>(As[cur ^ 1], a_km, ra);
            stash_tile<BN>(Bs[cur ^ 1], b_km, rb);
        }
        __syncthreads();
    }

    float* cbase = g.c + (int64_t)bz * g.M * g.N;
    const bool add_bias = g.bias != nullptr && gridDim.z == 1;
#pragma unroll
    for (int j = 0; j < TJ; j++) {
        const int64_t col = n0 + wn * (BN / 4) + j * 16 + (lane & 15);
        if (col >= g.N) continue;
        const float bv = add_bias ? g.bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                if (row >= g.M) continue;
                const float prev = (g.accumulate && gridDim.z == 1) ? cbase[row * g.N + col] : 0.f;
                cbase[row * g.N + col] = prev + (acc[i][j][r] + bv);
            }
        }
    }
}

// ---- the main tile kernel for n > 64: 128 x 128 outputs per workgroup of four wavefronts,
// each owning 64 x 64 (a 4 x 4 grid of 16x16 MFMA tiles); k staged through LDS 32 at a time
// (one or two buffers, BigCfg), the next stage's global loads in flight during the current MFMAs.  An
// operand whose rows run along k (a plain, b transposed) is staged as [row][k], one whose
// rows run along m or n (a transposed, b plain) as [k][row]: both are 16-byte copies, with
// no transposition on the way into LDS.  Both layouts are free of bank conflicts for the
// stores and the MFMA operand reads: a [row][k] tile (rows of 32 floats, no padding) is
// read 16 bytes per lane (four k at once, the contraction index permuted inside the stage as
// in gemm_f32_mfma), with the eight 16-byte chunks of row r stored in the order
// c ^ swz(r), so that 16 consecutive rows reading the same chunk hit different banks; a
// [k][row] tile is read one float per lane, its pitch putting the four lane groups' k rows
// 16 banks apart.
constexpr int kBigThreads = 256;
constexpr int TT = 128;                     // tile rows and columns
constexpr int TK2 = 32;                     // k per stage
constexpr int PITCH_RK = TK2;               // [row][k]
constexpr int PITCH_KR = TT + 4;            // [k][row]
constexpr int kStageFloats = TK2 * PITCH_KR;  // >= TT * PITCH_RK
constexpr int kEpPitch = 68;                   // epilogue rows: 64 columns + 4
constexpr int kEpFloats = 4 * 32 * kEpPitch;   // four wavefronts' 32-row epilogue blocks

// Stage buffers and workgroups per CU of one instance.  One buffer (two barriers per stage)
// lets three workgroups share a CU, so one's barriers, prologue and epilogue are covered by
// the others' MFMAs: 3-5% faster than two double-buffered workgroups.  Only a b^T keeps two
// buffers and two workgroups: three of its workgroups ran 6-7% slower, also in a build whose
// loop fitted the 168 registers without spilling.  (A fourth workgroup for a^T b gained 1%.)
template <bool AKM, bool BKM>
struct BigCfg {
    static constexpr int buffers = (AKM || BKM) ? 1 : 2;
    static constexpr int per_cu = 4 - buffers;
    static constexpr int lds_floats = 2 * buffers * kStageFloats > kEpFloats ? 2 * buffers * kStageFloats : kEpFloats;
};

// chunk order of a [row][k] row: a different permutation for each of 8 consecutive rows
// and for each parity among 16
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// This thread's four 16-byte pieces of one operand stage: rows row0 + 32q of a [row][k]
// tile (eight threads per 32-float row), or k rows kr0 + 8q of a [k][row] tile (32 threads
// per 128-float row).
template <bool KM>
__device__ __forceinline__ void big_fetch(const float* src, int64_t ld, int64_t o0, int64_t olim, int64_t k0,
                                          int64_t klim, bool fast, bool vec, v4f (&r)[4]) {
    const int t = threadIdx.x;
    if constexpr (!KM) {
        const int row = t >> 3, k4 = (t & 7) * 4;
        if (fast) {
            const float* p = src + (o0 + row) * ld + k0 + k4;
#pragma unroll
            for (int q = 0; q < 4; q++) r[q] = *reinterpret_cast<const v4f*>(p + (int64_t)(32 * q) * ld);
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t o = o0 + row + 32 * q;
                const float4 x = o < olim ? load4(src + o * ld, k0 + k4, klim, vec) : make_float4(0.f, 0.f, 0.f, 0.f);
                r[q] = v4f{x.x, x.y, x.z, x.w};
            }
        }
    } else {
        const int kr = t >> 5, c4 = (t & 31) * 4;
        if (fast) {
            const float* p = src + (k0 + kr) * ld + o0 + c4;
#pragma unroll
            for (int q = 0; q < 4; q++) r[q] = *reinterpret_cast<const v4f*>(p + (int64_t)(8 * q) * ld);
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t k = k0 + kr + 8 * q;
                const float4 x = k < klim ? load4(src + k * ld, o0 + c4, olim, vec) : make_float4(0.f, 0.f, 0.f, 0.f);
                r[q] = v4f{x.x, x.y, x.z, x.w};
            }
        }
    }
}

template <bool KM>
__device__ __forceinline__ void big_stash(float* lds, const v4f (&r)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int row = (t >> 3) + 32 * q;
        float* d = KM ? lds + ((t >> 5) + 8 * q) * PITCH_KR + (t & 31) * 4
                      : lds + row * PITCH_RK + 4 * ((t & 7) ^ swz(row));
        *reinterpret_cast<v4f*>(d) = r[q];
    }
}

// Operand values of one 16-wide tile (rows base .. base+15) for the four MFMA steps of a
// 16-deep half stage h: step t takes k = 16h + 4g + t in lane group g = lane / 16.
template <bool KM>
__device__ __forceinline__ void big_operand(const float* lds, int base, int h, int lane, float (&v)[4]) {
    const int r = lane & 15, kq = h * 16 + (lane >> 4) * 4;
    if constexpr (!KM) {
        const int row = base + r;
        const v4f x = *reinterpret_cast<const v4f*>(lds + row * PITCH_RK + 4 * ((kq >> 2) ^ swz(row)));
        v[0] = x[0];
        v[1] = x[1];
        v[2] = x[2];
        v[3] = x[3];
    } else {
#pragma unroll
        for (int t = 0; t < 4; t++) v[t] = lds[(kq + t) * PITCH_KR + base + r];
    }
}

// Pointers to this thread's four 16-byte pieces of an operand stage (see big_fetch) when
// the whole tile and k range are inside the matrix, and the distance to the next stage.
template <bool KM>
__device__ __forceinline__ int64_t fast_rows(const float* src, int64_t ld, int64_t o0, int64_t k0,
                                             const float* (&p)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 4; q++)
        p[q] = KM ? src + (k0 + (t >> 5) + 8 * q) * ld + o0 + (t & 31) * 4
                  : src + (o0 + (t >> 3) + 32 * q) * ld + k0 + (t & 7) * 4;
    return KM ? (int64_t)TK2 * ld : TK2;
}

__device__ __forceinline__ void fast_fetch(const float* (&p)[4], int64_t step, v4f (&r)[4]) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
        r[q] = *reinterpret_cast<const v4f*>(p[q]);
        p[q] += step;
    }
}

// The k loop of one tile: nk stages from kb through NB LDS buffers (with one, the stores of
// the next stage wait at a barrier for every wavefront's reads of the current one).  FAST:
// the tile and every stage lie inside the matrices, and rows are 16-byte aligned.
// Adds this thread's a values of one stage (rows row0 + 32q, k = k0 + 4 (t % 8) .. +3; see
// big_fetch) times gate_w to its four row sums (plain a only).
__device__ __forceinline__ void gate_stage(const float* gw, int64_t k0, int64_t klim, bool vec, const v4f (&ra)[4],
                                           float (&gs)[4]) {
    const float4 w = load4(gw, k0 + (threadIdx.x & 7) * 4, klim, vec);
#pragma unroll
    for (int q = 0; q < 4; q++) {
        gs[q] = fmaf(ra[q][0], w.x, gs[q]);
        gs[q] = fmaf(ra[q][1], w.y, gs[q]);
        gs[q] = fmaf(ra[q][2], w.z, gs[q]);
        gs[q] = fmaf(ra[q][3], w.w, gs[q]);
    }
}

template <bool AKM, bool BKM, bool FAST, int NB>
__device__ __forceinline__ void big_loop(const GemmArgs& g, float (*lds)[2][kStageFloats], int64_t m0, int64_t n0,
                                         int64_t kb, int64_t ke, bool a_vec, bool b_vec, v4f (&acc)[4][4],
                                         const float* gw = nullptr, float* gsp = nullptr) {
    // (gw == nullptr in every call of the plain instances: the gate code folds away)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (int)((ke - kb + TK2 - 1) / TK2);
    v4f ra[4], rb[4];
    const float* pa[4];
    const float* pb[4];
    const int64_t sa = fast_rows<AKM>(g.a, g.lda, m0, kb, pa);
    const int64_t sb = fast_rows<BKM>(g.b, g.ldb, n0, kb, pb);
#define GGA_BIG_FETCH(k0)                                                      \
    if constexpr (FAST) {                                                      \
        fast_fetch(pa, sa, ra);                                                \
        fast_fetch(pb, sb, rb);                                                \
    } else {                                                                   \
        big_fetch<AKM>(g.a, g.lda, m0, g.M, (k0), ke, false, a_vec, ra);       \
        big_fetch<BKM>(g.b, g.ldb, n0, g.N, (k0), ke, false, b_vec, rb);       \
    }
    float gs[4] = {0.f, 0.f, 0.f, 0.f};
    const bool gate = !AKM && gw != nullptr;
    const bool gw_vec = gate && (reinterpret_cast<uintptr_t>(gw) & 15) == 0;
    if (nk > 0) {
        GGA_BIG_FETCH(kb)
        if (gate) gate_stage(gw, kb, ke, gw_vec, ra, gs);
        big_stash<AKM>(lds[0][0], ra);
        big_stash<BKM>(lds[0][1], rb);
    }
    __syncthreads();
    for (int t = 0; t < nk; t++) {
        const int cur = NB == 2 ? (t & 1) : 0;
        if (t + 1 < nk) {
            GGA_BIG_FETCH(kb + (int64_t)(t + 1) * TK2)
        }
        const float* as = lds[cur][0];
        const float* bs = lds[cur][1];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            float af[4][4], bf[4][4];
#pragma unroll
            for (int i = 0; i < 4; i++) big_operand<AKM>(as, wm * 64 + i * 16, h, lane, af[i]);
#pragma unroll
            for (int j = 0; j < 4; j++) big_operand<BKM>(bs, wn * 64 + j * 16, h, lane, bf[j]);
#pragma unroll
            for (int st = 0; st < 4; st++)
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][st], bf[j][st], acc[i][j], 0, 0, 0);
        }
        if (t + 1 < nk) {
            if (gate) gate_stage(gw, kb + (int64_t)(t + 1) * TK2, ke, gw_vec, ra, gs);
            if constexpr (NB == 1) __syncthreads();
            big_stash<AKM>(lds[NB == 2 ? cur ^ 1 : 0][0], ra);
            big_stash<BKM>(lds[NB == 2 ? cur ^ 1 : 0][1], rb);
        }
        __syncthreads();
    }
#undef GGA_BIG_FETCH
    if (gate)
#pragma unroll
        for (int q = 0; q < 4; q++) gsp[q] += gs[q];
}

// The outer-product term's values for one lane of a 128 x 128 tile: its 16 rows (two halves
// of 8) and 4 columns.
struct R1Vals {
    float u[2][8];
    v4f w;
};

// Requested at the start of the kernel that takes the term, so the loads are long done when
// the epilogue uses them.
__device__ __forceinline__ R1Vals load_r1(const GemmArgs& g, int64_t m0, int64_t n0) {
    R1Vals r;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1, cl = lane & 15;
    const bool on = g.r1_row != nullptr;
    const int64_t col = n0 + wn * 64 + cl * 4;
#pragma unroll
    for (int e = 0; e < 4; e++) r.w[e] = on && col + e < g.N ? g.r1_col[col + e] : 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int it = 0; it < 8; it++) {
            const int64_t row = m0 + wm * 64 + hh * 32 + it * 4 + (lane >> 4);
            r.u[hh][it] = on && row < g.M ? g.r1_row[row] : 0.f;
        }
    return r;
}

// Epilogue of a 128 x 128 tile through LDS, 32 rows of the wavefront's 64 x 64 block at a
// time: the accumulators go to a private [32][68] region, then each row leaves as 16-byte
// stores, 16 lanes covering 64 consecutive columns.  R1: the outer-product term of GemmArgs
// (values from load_r1) is added when its pointers are set; only the instance that takes it
// compiles it.
template <bool R1 = false>
__device__ __forceinline__ void big_epilogue(const GemmArgs& g, float* lds_raw, const v4f (&acc)[4][4], int64_t m0,
                                             int64_t n0, uint32_t bz, const R1Vals* r1 = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    float* cbase = g.c + (int64_t)bz * g.M * g.N;
    const bool add_bias = g.bias != nullptr && gridDim.z == 1;
    const bool acc_in = g.accumulate && gridDim.z == 1;
    const bool add_r1 = R1 && g.r1_row != nullptr && gridDim.z == 1;
    const bool c_vec = (g.N % 4) == 0 && (reinterpret_cast<uintptr_t>(g.c) & 15) == 0 &&
                       (!add_bias || (reinterpret_cast<uintptr_t>(g.bias) & 15) == 0);
    constexpr int EP = kEpPitch;
    float* ep = lds_raw + wave * 32 * EP;
    const int g4 = (lane >> 4) * 4, cl = lane & 15;
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) ep[(ii * 16 + g4 + r) * EP + j * 16 + cl] = acc[2 * hh + ii][j][r];
        __syncthreads();
        const int64_t col = n0 + wn * 64 + cl * 4;
#pragma unroll
        for (int it = 0; it < 8; it++) {
            const int rl = it * 4 + (lane >> 4);
            const int64_t row = m0 + wm * 64 + hh * 32 + rl;
            if (row >= g.M) continue;
            const v4f v = *reinterpret_cast<const v4f*>(ep + rl * EP + cl * 4);
            float* dst = cbase + row * g.N + col;
            const float ur = R1 && add_r1 ? r1->u[hh][it] : 0.f;
            if (c_vec && col + 3 < g.N) {
                v4f o = v;
                if (add_bias) o += *reinterpret_cast<const v4f*>(g.bias + col);
                if (R1 && add_r1) {
#pragma unroll
                    for (int e = 0; e < 4; e++) o[e] = fmaf(ur, r1->w[e], o[e]);
                }
                if (acc_in) o = *reinterpret_cast<const v4f*>(dst) + o;
                *reinterpret_cast<v4f*>(dst) = o;
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (col + e >= g.N) continue;
                    float o = v[e] + (add_bias ? g.bias[col + e] : 0.f);
                    if (R1 && add_r1) o = fmaf(ur, r1->w[e], o);
                    dst[e] = acc_in ? dst[e] + o : o;
                }
            }
        }
    }
}

template <bool AKM, bool BKM>
__global__ __launch_bounds__(kBigThreads, (BigCfg<AKM, BKM>::per_cu)) void gemm_f32_big(GemmArgs g) {
    using Cfg = BigCfg<AKM, BKM>;
    __shared__ float lds_raw[Cfg::lds_floats];
    // [buffer][operand]; the epilogue reuses the same memory
    float(*lds)[2][kStageFloats] = reinterpret_cast<float(*)[2][kStageFloats]>(lds_raw);
    const uint32_t gxy = gridDim.x * gridDim.y;
    const uint32_t tl = xcd_order(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gxy * gridDim.z);
    const uint32_t bz = tl / gxy, by = (tl % gxy) / gridDim.x, bx = tl % gridDim.x;
    const int64_t m0 = (int64_t)by * TT, n0 = (int64_t)bx * TT;
    const int64_t kb = (int64_t)bz * g.kchunk;
    const int64_t ke = kb + g.kchunk < g.K ? kb + g.kchunk : g.K;
    const bool a_vec = (g.lda % 4) == 0 && (reinterpret_cast<uintptr_t>(g.a) & 15) == 0;
    const bool b_vec = (g.ldb % 4) == 0 && (reinterpret_cast<uintptr_t>(g.b) & 15) == 0;
    const bool fast = a_vec && b_vec && m0 + TT <= g.M && n0 + TT <= g.N && (ke - kb) % TK2 == 0;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (fast)
        big_loop<AKM, BKM, true, Cfg::buffers>(g, lds, m0, n0, kb, ke, a_vec, b_vec, acc);
    else
        big_loop<AKM, BKM, false, Cfg::buffers>(g, lds, m0, n0, kb, ke, a_vec, b_vec, acc);

    big_epilogue(g, lds_raw, acc, m0, n0, bz);
}

// Products with segmented operands (plain a and b), two workgroups per CU.
//
// Column segments (gemm_f32_seg_cols): each seg_len-wide column range of op(b) and c is its
// own pair of matrices; with gate_out, the workgroups of column tile 0 also form
// a . gate_w for their rows from the a values they load.
__global__ __launch_bounds__(kBigThreads, 2) void gemm_f32_seg_cols(GemmArgs g) {
    using Cfg = BigCfg<false, true>;
    __shared__ float lds_raw[Cfg::lds_floats];
    float(*lds)[2][kStageFloats] = reinterpret_cast<float(*)[2][kStageFloats]>(lds_raw);
    const uint32_t gxy = gridDim.x * gridDim.y;
    const uint32_t tl = xcd_order(blockIdx.x + gridDim.x * blockIdx.y, gxy);
    const uint32_t by = tl / gridDim.x, bx = tl % gridDim.x;
    const int64_t m0 = (int64_t)by * TT;
    const int sg = (int)(((int64_t)bx * TT) / g.seg_len);
    const int64_t n0 = (int64_t)bx * TT - (int64_t)sg * g.seg_len;
    GemmArgs gv = g;  // the tile's own matrices
    gv.b = g.seg_b[sg];
    gv.c = g.seg_c[sg];
    gv.N = g.seg_len;
    gv.ldb = g.seg_len;
    const bool do_gate = g.gate_out != nullptr && bx == 0;
    float gsum[4] = {0.f, 0.f, 0.f, 0.f};
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const bool a_vec = (gv.lda % 4) == 0 && (reinterpret_cast<uintptr_t>(gv.a) & 15) == 0;
    const bool b_vec = (gv.ldb % 4) == 0 && (reinterpret_cast<uintptr_t>(gv.b) & 15) == 0;
    const bool fast = a_vec && b_vec && m0 + TT <= gv.M && n0 + TT <= gv.N && gv.K % TK2 == 0;
    const float* gw = do_gate ? g.gate_w : nullptr;
    if (fast)
        big_loop<false, true, true, Cfg::buffers>(gv, lds, m0, n0, 0, gv.K, a_vec, b_vec, acc, gw, gsum);
    else
        big_loop<false, true, false, Cfg::buffers>(gv, lds, m0, n0, 0, gv.K, a_vec, b_vec, acc, gw, gsum);
    if (do_gate) {
        // the eight threads of a row segment hold its eight k chunks: a fixed butterfly
#pragma unroll
        for (int q = 0; q < 4; q++) {
            float v = gsum[q];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            const int64_t row = m0 + (threadIdx.x >> 3) + 32 * q;
            if ((threadIdx.x & 7) == 0 && row < g.M) g.gate_out[row] = v + g.gate_b;
        }
    }
    big_epilogue(gv, lds_raw, acc, m0, n0, 0);
}

// k segments (gemm_f32_seg_k<S>): the k range [s seg_len, (s+1) seg_len) of a and b is the
// pair seg_a[s] [M, seg_len], seg_b[s] [seg_len, N]; the segments run in order into the same
// accumulators, so the sum is the one a single product over the concatenated k would form.
template <int S>
__global__ __launch_bounds__(kBigThreads, 2) void gemm_f32_seg_k(GemmArgs g) {
    using Cfg = BigCfg<false, true>;
    __shared__ float lds_raw[Cfg::lds_floats];
    float(*lds)[2][kStageFloats] = reinterpret_cast<float(*)[2][kStageFloats]>(lds_raw);
    const uint32_t gxy = gridDim.x * gridDim.y;
    const uint32_t tl = xcd_order(blockIdx.x + gridDim.x * blockIdx.y, gxy);
    const uint32_t by = tl / gridDim.x, bx = tl % gridDim.x;
    const int64_t m0 = (int64_t)by * TT, n0 = (int64_t)bx * TT;
    const R1Vals r1 = load_r1(g, m0, n0);  // zeros when the term is absent
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    bool fast = m0 + TT <= g.M && n0 + TT <= g.N && g.seg_len % TK2 == 0 && g.seg_len % 4 == 0 && g.ldb % 4 == 0;
#pragma unroll
    for (int kp = 0; kp < S; kp++)
        fast = fast && (reinterpret_cast<uintptr_t>(g.seg_a[kp]) & 15) == 0 &&
               (reinterpret_cast<uintptr_t>(g.seg_b[kp]) & 15) == 0;
    if (fast) {
#pragma unroll
        for (int kp = 0; kp < S; kp++) {
            GemmArgs gk = g;
            gk.a = g.seg_a[kp];
            gk.b = g.seg_b[kp];
            gk.K = g.seg_len;
            gk.lda = g.seg_len;
            big_loop<false, true, true, Cfg::buffers>(gk, lds, m0, n0, 0, g.seg_len, true, true, acc);
        }
    } else {
#pragma unroll
        for (int kp = 0; kp < S; kp++) {
            GemmArgs gk = g;
            gk.a = g.seg_a[kp];
            gk.b = g.seg_b[kp];
            gk.K = g.seg_len;
            gk.lda = g.seg_len;
            const bool a_vec = (g.seg_len % 4) == 0 && (reinterpret_cast<uintptr_t>(gk.a) & 15) == 0;
            const bool b_vec = (gk.ldb % 4) == 0 && (reinterpret_cast<uintptr_t>(gk.b) & 15) == 0;
            big_loop<false, true, false, Cfg::buffers>(gk, lds, m0, n0, 0, g.seg_len, a_vec, b_vec, acc);
        }
    }
    big_epilogue<true>(g, lds_raw, acc, m0, n0, 0, &r1);
}

// c[i,j] += u[i] v[j] over an n x d matrix (the outer-product term of the k-segmented dX
// product when that product cannot take it in its epilogue).
__global__ __launch_bounds__(256) void rank1_add(int32_t n, int32_t d, const float* __restrict__ u,
                                                 const float* __restrict__ v, float* __restrict__ c) {
    const int64_t total = (int64_t)n * d;
    for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < total; x += (int64_t)gridDim.x * blockDim.x)
        c[x] = fmaf(u[x / d], v[x % d], c[x]);
}

// gate[i] = x[i,:] . w + b, one wavefront per row, a fixed butterfly over the lanes (the
// projections' path when the layer width is not a multiple of the 128-wide tile).
__global__ __launch_bounds__(256) void gate_logit_kernel(int32_t n, int32_t d, const float* __restrict__ x,
                                                         const float* __restrict__ w, float b,
                                                         float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const int64_t i = blockIdx.x * 4ll + (threadIdx.x >> 6);
    if (i >= n) return;
    float t = 0.f;
    for (int j = lane; j < d; j += 64) t = fmaf(x[i * d + j], w[j], t);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) t += __shfl_xor(t, o, 64);
    if (lane == 0) gate[i] = t + b;
}

// dst[c][r] = src[r][c] for a rows x cols matrix, through a 32 x 32 LDS tile padded by one
// column (the column reads of the second half then hit distinct banks).
__global__ __launch_bounds__(256) void transpose_f32(const float* __restrict__ src, int32_t rows, int32_t cols,
                                                     float* __restrict__ dst) {
    __shared__ float t[32][33];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * 32, r0 = (int64_t)blockIdx.y * 32;
    for (int i = ty; i < 32; i += 8) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) t[i][tx] = src[r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) dst[c * rows + r] = t[tx][i];
    }
}

// c = (c if accumulating) + (sum over the splits of the partial products (in split order) + bias).  A workgroup of
// 16 wavefronts owns 64 consecutive outputs: wavefront w adds splits w, w+16, ... and the
// 16 running sums are then added in wavefront order.
__global__ __launch_bounds__(1024) void splitk_reduce(const float* __restrict__ part, int splits, int64_t mn,
                                                      int32_t N, const float* __restrict__ bias, int accumulate,
                                                      float* __restrict__ c) {
    __shared__ float sm[16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * 64 + lane;
    float s = 0.f;
    if (i < mn) {
        // eight of the wavefront's splits are requested at a time and added in split order
        // (the same sums as one at a time)
        int z = wave;
        for (; z + 7 * 16 < splits; z += 8 * 16) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = part[(int64_t)(z + 16 * j) * mn + i];
#pragma unroll
            for (int j = 0; j < 8; j++) s += v[j];
        }
        for (; z < splits; z += 16) s += part[(int64_t)z * mn + i];
    }
    sm[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && i < mn) {
        float t = 0.f;
        for (int w = 0; w < 16; w++) t += sm[w][lane];
        const float prev = accumulate ? c[i] : 0.f;
        c[i] = prev + (t + (bias ? bias[i % N] : 0.f));
    }
}

// ---- tall products with all of op(b) in LDS (k, n <= 128, multiples of 16, k*n <= 8192,
// plain a): each workgroup stages op(b) once as [n][k] (rows padded by 4 floats, so the
// 16-byte reads of 16 consecutive n rows hit distinct banks) and its eight wavefronts take
// one 16-row tile of a each (measured best of 1-8 tiles and 4 or 8 wavefronts).  In 16-deep chunk h, lane (r = lane%16, g = lane/16) holds
// a[row r][16h + 4g .. +3] (one 16-byte load) and b[16h + 4g .. +3][16j + r] (one LDS
// read), MFMA step t taking k = 16h + 4g + t; lane l ends with c[4g + i][16j + r].  The next
// tile's a rows are loaded during the current tile's MFMAs.
constexpr int kStreamTiles = 1;  // 16-row tiles per wavefront
constexpr int kStreamWaves = 8;  // wavefronts per workgroup (sharing one staged op(b))
constexpr int kStreamThreads = 64 * kStreamWaves;

template <int KC, int NT>
__global__ __launch_bounds__(kStreamThreads) void gemm_stream(GemmArgs g) {
    constexpr int K = KC * 16, N = NT * 16, PB = K + 4;
    __shared__ float bt[N * PB];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const int64_t t0 = ((int64_t)blockIdx.x * kStreamWaves + wave) * kStreamTiles;
    // op(b) in its memory order, 16 bytes per load, requested first (the staging stores wait
    // for these loads only, not for the a rows requested after them)
    constexpr int NV = K * N / 4, PER = (NV + kStreamThreads - 1) / kStreamThreads;
    v4f sv[PER];
#pragma unroll
    for (int q = 0; q < PER; q++) {
        const int x = threadIdx.x + kStreamThreads * q;
        if (x < NV) sv[q] = *reinterpret_cast<const v4f*>(g.b + 4 * x);
    }
    // every tile's a rows are requested before any tile is multiplied, so the loads of the
    // later tiles arrive while the earlier ones are multiplied; rows past the end re-read
    // the last row (never stored), so no load is conditional
    v4f at[kStreamTiles][KC];
#pragma unroll
    for (int tt = 0; tt < kStreamTiles; tt++) {
        const int64_t row = min((t0 + tt) * 16 + r, (int64_t)g.M - 1);
#pragma unroll
        for (int h = 0; h < KC; h++) at[tt][h] = *reinterpret_cast<const v4f*>(g.a + row * K + 16 * h + 4 * gq);
    }
#pragma unroll
    for (int q = 0; q < PER; q++) {
        const int x = threadIdx.x + kStreamThreads * q;
        if (x >= NV) continue;
        if (g.trans_b) {  // b [N][K]: four consecutive k of row j
            const int j = 4 * x / K, kk = 4 * x % K;
            *reinterpret_cast<v4f*>(bt + j * PB + kk) = sv[q];
        } else {  // b [K][N]: four consecutive n of row kk
            const int kk = 4 * x / N, j0 = 4 * x % N;
#pragma unroll
            for (int e = 0; e < 4; e++) bt[(j0 + e) * PB + kk] = sv[q][e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kStreamTiles; tt++) {
        const int64_t tile = t0 + tt;
        if (tile * 16 >= g.M) break;
        v4f acc[NT];
#pragma unroll
        for (int j = 0; j < NT; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < KC; h++) {
            v4f b[NT];
#pragma unroll
            for (int j = 0; j < NT; j++) b[j] = *reinterpret_cast<const v4f*>(bt + (16 * j + r) * PB + 16 * h + 4 * gq);
            // consecutive MFMAs go to different accumulators
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int j = 0; j < NT; j++)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(at[tt][h][t], b[j][t], acc[j], 0, 0, 0);
        }
        if (g.bias) {
#pragma unroll
            for (int j = 0; j < NT; j++) acc[j] += g.bias[16 * j + r];
        }
        if (g.accumulate) {  // every read of c before any write
            v4f old[NT];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t row = min(tile * 16 + 4 * gq + i, (int64_t)g.M - 1);
#pragma unroll
                for (int j = 0; j < NT; j++) old[j][i] = g.c[row * N + 16 * j + r];
            }
#pragma unroll
            for (int j = 0; j < NT; j++) acc[j] = old[j] + acc[j];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t row = tile * 16 + 4 * gq + i;
            if (row >= g.M) continue;
            float* dst = g.c + row * N + r;
#pragma unroll
            for (int j = 0; j < NT; j++) dst[16 * j] = acc[j][i];
        }
    }
}

// ---- skinny shapes, where a 128-row MFMA tile would mostly compute padding

// element (r, kk) of op(a) and (kk, j) of op(b)
__device__ __forceinline__ float op_a(const GemmArgs& g, int64_t r, int64_t kk) {
    return g.trans_a ? g.a[kk * g.M + r] : g.a[r * g.K + kk];
}
__device__ __forceinline__ float op_b(const GemmArgs& g, int64_t kk, int64_t j) {
    return g.trans_b ? g.b[j * g.K + kk] : g.b[kk * g.N + j];
}

// Few outputs of a transposed-A product (c = a^T b, a stored [K][M], b [K][N]; M, N <= 32)
// over a long k: workgroup z sums its k range into part[z][M][N].  Rows of a and b come
// through LDS 128 at a time (coalesced), the next tile's loads issued before the current
// one is used; with M*N < 256 each output's rows are split into interleaved streams added
// in stream order.
__global__ __launch_bounds__(256) void gemm_small_out(GemmArgs g, float* __restrict__ part) {
    constexpr int TR = 128, PER = TR * 32 / 256;
    __shared__ float as[TR * 32], bs[TR * 32];
    __shared__ float sm[256];
    const int t = threadIdx.x;
    const int M = g.M, N = g.N, mn = M * N;
    const int64_t kb = (int64_t)blockIdx.x * g.kchunk;
    const int64_t ke = kb + g.kchunk < g.K ? kb + g.kchunk : g.K;
    const int reps = mn < 256 ? 256 / mn : 1;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float ra[PER], rb[PER];
    auto fetch = [&](int64_t r0) {
        const int rows = (int)(ke - r0 < TR ? ke - r0 : TR);
#pragma unroll
        for (int q = 0; q < PER; q++) {
            const int x = t + 256 * q;
            ra[q] = x < rows * M ? g.a[r0 * M + x] : 0.f;
            rb[q] = x < rows * N ? g.b[r0 * N + x] : 0.f;
        }
    };
    if (kb < ke) fetch(kb);
    for (int64_t r0 = kb; r0 < ke; r0 += TR) {
        const int rows = (int)(ke - r0 < TR ? ke - r0 : TR);
#pragma unroll
        for (int q = 0; q < PER; q++) {
            as[t + 256 * q] = ra[q];
            bs[t + 256 * q] = rb[q];
        }
        __syncthreads();
        if (r0 + TR < ke) fetch(r0 + TR);
        if (mn < 256) {
            if (t < reps * mn) {
                const int o = t % mn, rs = t / mn;
                const int i = o / N, j = o % N;
                for (int r = rs; r < rows; r += reps) acc[0] = fmaf(as[r * M + i], bs[r * N + j], acc[0]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int o = t + 256 * q;
                if (o < mn) {
                    const int i = o / N, j = o % N;
                    for (int r = 0; r < rows; r++) acc[q] = fmaf(as[r * M + i], bs[r * N + j], acc[q]);
                }
            }
        }
        __syncthreads();
    }
    float* out = part + (int64_t)blockIdx.x * mn;
    if (mn < 256) {
        sm[t] = acc[0];
        __syncthreads();
        if (t < mn) {
            float s = 0.f;
            for (int r = 0; r < reps; r++) s += sm[r * mn + t];
            out[t] = s;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; q++)
            if (t + 256 * q < mn) out[t + 256 * q] = acc[q];
    }
}

// Narrow contraction (K, N <= 64): a workgroup owns 64 output rows; their op(a) rows and
// op(b) are staged in LDS with coalesced loads, and thread t computes outputs t, t+256, ...
// of the 64 x N block (so stores are coalesced), summing k in order.
// Short rows (k, n <= 32): one thread per output row, op(b) in LDS (read by broadcast), the
// row of op(a) in registers; each output sums over k in order, as gemm_narrow does.  When a
// wavefront's 64 rows lie inside the matrices with 16-byte rows (plain a), the rows move
// through a wavefront-private LDS block both ways, so every global access is a contiguous
// 16-byte-per-lane run (measured faster than per-thread rows on either side alone for
// k = 16, n = 8 and k = 8, n = 16); otherwise each thread reads and writes its own row.
template <int KP, int NP>
__global__ __launch_bounds__(256) void gemm_rows(GemmArgs g) {
    constexpr int PA = KP + 4, PC = NP + 4;  // padded rows: 16-byte reads of 8 lanes hit distinct banks
    __shared__ float bs[KP * NP];
    __shared__ float stage[4][64 * (PA > PC ? PA : PC)];
    const int K = g.K, N = g.N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
    const int64_t r = r0 + lane;
    // (K > 0: an empty a has no first element for the clamped loads below to re-read)
    const bool tile = !g.trans_a && K > 0 && K % 4 == 0 && N % 4 == 0 && r0 + 64 <= g.M &&
                      (reinterpret_cast<uintptr_t>(g.a) & 15) == 0 && (reinterpret_cast<uintptr_t>(g.c) & 15) == 0;
    // the wavefront's 64 rows of K floats are requested first, 4 at a time, all in flight
    // together and during the op(b) staging (positions past 16 K re-read the first one)
    v4f v[KP / 4];
    if (tile) {
        const float* src = g.a + r0 * K;
#pragma unroll
        for (int q = 0; q < KP / 4; q++) {
            const int x = lane + 64 * q;
            v[q] = *reinterpret_cast<const v4f*>(src + 4 * (x < 16 * K ? x : 0));
        }
    }
    for (int x = threadIdx.x; x < K * N; x += 256) bs[x] = op_b(g, x / N, x % N);
    float* st = stage[wave];
    float a[KP];
    __syncthreads();  // bs complete; from here on each wavefront works alone
    if (r >= g.M) return;
    if (tile) {
#pragma unroll
        for (int q = 0; q < KP / 4; q++) {
            const int x = lane + 64 * q;
            if (x < 16 * K) *reinterpret_cast<v4f*>(st + (4 * x / K) * PA + (4 * x) % K) = v[q];
        }
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < KP / 4; q++) {
            const v4f x = q * 4 < K ? *reinterpret_cast<const v4f*>(st + lane * PA + 4 * q) : v4f{0.f, 0.f, 0.f, 0.f};
            a[4 * q] = x[0];
            a[4 * q + 1] = x[1];
            a[4 * q + 2] = x[2];
            a[4 * q + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KP; kk++) a[kk] = kk < K ? op_a(g, r, kk) : 0.f;
    }
    float o[NP];
#pragma unroll
    for (int j = 0; j < NP; j++) {
        float acc = 0.f;
#pragma unroll
        for (int kk = 0; kk < KP; kk++)
            if (kk < K && j < N) acc = fmaf(a[kk], bs[kk * N + j], acc);
        o[j] = acc + (g.bias && j < N ? g.bias[j] : 0.f);
    }
    if (tile) {
        // the wavefront's rows leave through LDS (its A rows were all read above)
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < NP / 4; q++)
            if (q * 4 < N) *reinterpret_cast<v4f*>(st + lane * PC + 4 * q) = v4f{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
        wave_lds_sync();
        float* dst = g.c + r0 * N;
#pragma unroll
        for (int q = 0; q < NP / 4; q++) {
            const int x = lane + 64 * q;
            if (x >= 16 * N) continue;
            v4f v = *reinterpret_cast<const v4f*>(st + (4 * x / N) * PC + (4 * x) % N);
            if (g.accumulate) v = *reinterpret_cast<const v4f*>(dst + 4 * x) + v;
            *reinterpret_cast<v4f*>(dst + 4 * x) = v;
        }
        return;
    }
    float* c = g.c + r * N;
#pragma unroll
    for (int j = 0; j < NP; j++)
        if (j < N) c[j] = (g.accumulate ? c[j] : 0.f) + o[j];
}

// Few outputs (m, n <= 16) of a transposed-a product c = a^T b over a long k (a stored
// [K][M], b [K][N]) on the matrix cores: one 16 x 16 tile, each MFMA taking four rows of k
// (lane l holds a[r + l/16][l%16] and b[r + l/16][l%16]: a wave-wide load of four
// consecutive rows each).  Workgroup z covers its fixed k range; wavefront w takes the
// 64-row blocks kb + 64 (4 i + w), block row 4u + kq going to accumulation chain u % 4; the
// four chains are added in chain order, and the four wavefronts in wavefront order into
// part[z][M][N].
__global__ __launch_bounds__(256) void gemm_outer(GemmArgs g, float* __restrict__ part) {
    __shared__ float sm[4][256];
    const int M = g.M, N = g.N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int64_t kb = (int64_t)blockIdx.x * g.kchunk;
    const int64_t ke = kb + g.kchunk < g.K ? kb + g.kchunk : g.K;
    v4f acc[4];
#pragma unroll
    for (int u = 0; u < 4; u++) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int64_t r0 = kb + 64 * wave; r0 < ke; r0 += 256) {
        float av[16], bv[16];  // 64 rows in flight per wavefront
#pragma unroll
        for (int u = 0; u < 16; u++) {
            const int64_t r = r0 + 4 * u + kq;
            const bool ok = r < ke;
            av[u] = ok && col < M ? g.a[r * M + col] : 0.f;
            bv[u] = ok && col < N ? g.b[r * N + col] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; u++)
            acc[u & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u], acc[u & 3], 0, 0, 0);
    }
    const v4f t = ((acc[0] + acc[1]) + acc[2]) + acc[3];
    // acc element e of lane l is c[4 (l / 16) + e][l % 16]
#pragma unroll
    for (int e = 0; e < 4; e++) sm[wave][(4 * kq + e) * 16 + col] = t[e];
    __syncthreads();
    float* out = part + (int64_t)blockIdx.x * M * N;
    for (int x = threadIdx.x; x < M * N; x += 256) {
        const int i = x / N, j = x % N;
        out[x] = ((sm[0][i * 16 + j] + sm[1][i * 16 + j]) + sm[2][i * 16 + j]) + sm[3][i * 16 + j];
    }
}

__global__ __launch_bounds__(256) void gemm_narrow(GemmArgs g) {
    __shared__ float as[64 * 65], bs[64 * 64];
    const int K = g.K, N = g.N;
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int rows = (int)(g.M - r0 < 64 ? g.M - r0 : 64);
    for (int x = threadIdx.x; x < K * N; x += 256) bs[x] = op_b(g, x / N, x % N);
    if (g.trans_a) {  // a stored [K][M]: rows of the tile are columns, k-major
        for (int x = threadIdx.x; x < K * 64; x += 256) {
            const int kk = x / 64, rr = x % 64;
            if (rr < rows) as[rr * 65 + kk] = g.a[(int64_t)kk * g.M + r0 + rr];
        }
    } else {  // the tile is one contiguous block of rows * K floats
        for (int x = threadIdx.x; x < rows * K; x += 256) as[(x / K) * 65 + x % K] = g.a[r0 * K + x];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < rows * N; o += 256) {
        const int rr = o / N, j = o % N;
        float acc = 0.f;
        for (int kk = 0; kk < K; kk++) acc = fmaf(as[rr * 65 + kk], bs[kk * N + j], acc);
        const int64_t ci = (r0 + rr) * N + j;
        const float prev = g.accumulate ? g.c[ci] : 0.f;
        g.c[ci] = prev + (acc + (g.bias ? g.bias[j] : 0.f));
    }
}

struct Split {
    int splits;
    int32_t kchunk;
};

// Few outputs and a long k: the small-output kernel over fixed k ranges of at least 1024
// (at most 2048 ranges); a transposed a, plain b.
bool small_out_shape(int32_t m, int32_t k, int32_t n) { return m <= 32 && n <= 32 && k > 4096; }

Split small_out_split(int32_t k) {
    int64_t kc = ((int64_t)k + 2047) / 2048;
    if (kc < 1024) kc = 1024;
    Split s;
    s.kchunk = (int32_t)kc;
    s.splits = (int)(((int64_t)k + kc - 1) / kc);
    return s;
}

bool narrow(int32_t k, int32_t n) { return k <= 64 && n <= 64; }

// Tall products whose whole op(b) fits the streaming kernel's LDS block.
bool stream_shape(int32_t m, int32_t k, int32_t n) {
    return m >= 1024 && k >= 16 && k % 16 == 0 && n % 16 == 0 && k <= 128 && n <= 128 && k * n <= 8192 &&
           !narrow(k, n);
}

// The register-row paths: short rows, or few outputs.
bool short_rows(int32_t k, int32_t n) { return k <= 32 && n <= 32; }
bool outer_shape(int32_t m, int32_t n) { return m <= 16 && n <= 16; }

// k ranges of the outer-product path: at least 4096 rows each, at most 1024 ranges (never
// more ranges than small_out_split gives, so the same workspace holds the partials).
Split outer_split(int32_t k) {
    int64_t kc = ((int64_t)k + 1023) / 1024;
    if (kc < 4096) kc = 4096;
    Split s;
    s.kchunk = (int32_t)kc;
    s.splits = (int)(((int64_t)k + kc - 1) / kc);
    return s;
}

int pow2_at_least4(int x) {
    int p = 4;
    while (p < x) p <<= 1;
    return p;
}

int pick_bn(int32_t n) { return n <= 64 ? 64 : 128; }

// Output tiles below 512: split k so that about 2048 workgroups run, each with at least 256
// values of k (a fixed function of the shape, so the summation order is too).
Split pick_split(int32_t m, int32_t k, int32_t n) {
    const int bn = pick_bn(n);
    const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + bn - 1) / bn);
    Split s{1, k};
    if (tiles < 512 && k > 1024) {
        // one round of resident workgroups in all: 512 for outputs of at most four tiles, 768
        // (three 128 x 128 workgroups per CU) for larger ones.  Against 2048: 4-9% faster on
        // [128 x 170000]^T [170000 x 64] and [256 x 262144]^T [262144 x 256], 0-11% on the
        // 256 x 768, 256 x 512, 512 x 512 and 512 x 1536 outputs (512 there was slower)
        const int64_t target = tiles <= 4 ? 512 : 768;
        int64_t want = (target + tiles - 1) / tiles;
        int64_t by_k = k / 256;
        int64_t sp = want < by_k ? want : by_k;
        if (sp > 1024) sp = 1024;
        if (sp > 1) {
            int64_t kc = (k + sp - 1) / sp;
            kc = (kc + 31) / 32 * 32;  // whole stages of either tile kernel
            s.kchunk = (int32_t)kc;
            s.splits = (int)((k + kc - 1) / kc);
        }
    }
    if (s.kchunk < 1) s.kchunk = 1;
    return s;
}

// a b^T with a tall a and a small b (a layer's weight): b is first transposed into the
// workspace and the product runs as a b, whose tile kernel keeps three workgroups on a CU
// where a b^T's keeps two.  Both feed the matrix cores the same k order, so the results
// are the same bits.
bool tall_abt(int32_t m, int32_t k, int32_t n) {
    return m >= 4096 && n > 64 && k >= 32 && (int64_t)k * n <= ((int64_t)1 << 22) && !narrow(k, n) &&
           !stream_shape(m, k, n) && pick_split(m, k, n).splits == 1;
}

}  // namespace
}  // namespace gga

using namespace gga;

extern "C" size_t gga_linear_workspace(int32_t m, int32_t k, int32_t n) {
    if (m < 0 || k < 0 || n < 0) return 0;
    const Split s = pick_split(m, k, n);
    size_t need = s.splits <= 1 ? 0 : align_up((size_t)s.splits * m * n * sizeof(float), 256);
    if (small_out_shape(m, k, n)) {  // (the choice also depends on the transposes)
        const size_t so = align_up((size_t)small_out_split(k).splits * m * n * sizeof(float), 256);
        need = so > need ? so : need;
    }
    if (tall_abt(m, k, n)) {  // (used only when b is transposed; the query does not know)
        const size_t bt = align_up((size_t)k * n * sizeof(float), 256);
        need = bt > need ? bt : need;
    }
    return need;
}

namespace {

int linear_impl(int32_t m, int32_t k, int32_t n, int32_t trans_a, int32_t trans_b, const float* a, const float* b,
                const float* bias, float* c, int accumulate, void* ws, size_t ws_bytes, void* stream) {
    if (m < 0 || k < 0 || n < 0) return GGA_EINVAL;
    if (m == 0 || n == 0) return GGA_OK;
    if (!c || (k > 0 && (!a || !b))) return GGA_EINVAL;
    if ((int64_t)m * n >= ((int64_t)1 << 40)) return GGA_ERANGE;
    hipStream_t s = as_stream(stream);
    const size_t need = gga_linear_workspace(m, k, n);
    if (ws_bytes < need || (need > 0 && !ws)) return GGA_EWORKSPACE;
    const bool so_path = small_out_shape(m, k, n) && trans_a && !trans_b;
    if (so_path || narrow(k, n)) {
        GemmArgs g{};
        g.a = a;
        g.b = b;
        g.bias = bias;
        g.c = c;
        g.M = m;
        g.K = k;
        g.N = n;
        g.trans_a = trans_a != 0;
        g.trans_b = trans_b != 0;
        g.accumulate = accumulate;
        if (so_path) {
            const bool outer = outer_shape(m, n);
            const Split so = outer ? outer_split(k) : small_out_split(k);
            g.kchunk = so.kchunk;
            float* part = static_cast<float*>(ws);
            if (!outer) {
                gemm_small_out<<<(unsigned)so.splits, 256, 0, s>>>(g, part);
            } else {
                gemm_outer<<<(unsigned)so.splits, 256, 0, s>>>(g, part);
            }
            const int64_t mn = (int64_t)m * n;
            splitk_reduce<<<(unsigned)((mn + 63) / 64), 1024, 0, s>>>(part, so.splits, mn, n, bias, accumulate, c);
        } else if (short_rows(k, n)) {
            const int64_t blocks = ((int64_t)m + 255) / 256;
            if (blocks >= ((int64_t)1 << 31)) return GGA_ERANGE;
            const int kp = pow2_at_least4(k), np = pow2_at_least4(n);
#define GGA_ROWS(KP_, NP_) \
    if (kp == KP_ && np == NP_) gemm_rows<KP_, NP_><<<(unsigned)blocks, 256, 0, s>>>(g);
            GGA_ROWS(4, 4) GGA_ROWS(4, 8) GGA_ROWS(4, 16) GGA_ROWS(4, 32) GGA_ROWS(8, 4) GGA_ROWS(8, 8)
            GGA_ROWS(8, 16) GGA_ROWS(8, 32) GGA_ROWS(16, 4) GGA_ROWS(16, 8) GGA_ROWS(16, 16) GGA_ROWS(16, 32)
            GGA_ROWS(32, 4) GGA_ROWS(32, 8) GGA_ROWS(32, 16) GGA_ROWS(32, 32)
#undef GGA_ROWS
        } else {
            const int64_t blocks = ((int64_t)m + 63) / 64;
            if (blocks >= ((int64_t)1 << 31)) return GGA_ERANGE;
            gemm_narrow<<<(unsigned)blocks, 256, 0, s>>>(g);
        }
        return launch_status();
    }
    if (!trans_a && stream_shape(m, k, n) && (reinterpret_cast<uintptr_t>(a) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(b) & 15) == 0) {
        GemmArgs g{};
        g.a = a;
        g.b = b;
        g.bias = bias;
        g.c = c;
        g.M = m;
        g.K = k;
        g.N = n;
        g.trans_b = trans_b != 0;
        g.accumulate = accumulate;
        const int64_t tiles = ((int64_t)m + 15) / 16;
        const int64_t blocks = (tiles + kStreamWaves * kStreamTiles - 1) / (kStreamWaves * kStreamTiles);
        const int kc = k / 16, nt = n / 16;
#define GGA_STREAM(KC_, NT_) \
    else if (kc == KC_ && nt == NT_) gemm_stream<KC_, NT_><<<(unsigned)blocks, kStreamThreads, 0, s>>>(g);
        if (false) {
        }
        GGA_STREAM(1, 5) GGA_STREAM(1, 6) GGA_STREAM(1, 7) GGA_STREAM(1, 8)
        GGA_STREAM(2, 5) GGA_STREAM(2, 6) GGA_STREAM(2, 7) GGA_STREAM(2, 8)
        GGA_STREAM(3, 5) GGA_STREAM(3, 6) GGA_STREAM(3, 7) GGA_STREAM(3, 8)
        GGA_STREAM(4, 5) GGA_STREAM(4, 6) GGA_STREAM(4, 7) GGA_STREAM(4, 8)
        GGA_STREAM(5, 1) GGA_STREAM(5, 2) GGA_STREAM(5, 3) GGA_STREAM(5, 4) GGA_STREAM(5, 5) GGA_STREAM(5, 6)
        GGA_STREAM(6, 1) GGA_STREAM(6, 2) GGA_STREAM(6, 3) GGA_STREAM(6, 4) GGA_STREAM(6, 5)
        GGA_STREAM(7, 1) GGA_STREAM(7, 2) GGA_STREAM(7, 3) GGA_STREAM(7, 4)
        GGA_STREAM(8, 1) GGA_STREAM(8, 2) GGA_STREAM(8, 3) GGA_STREAM(8, 4)
#undef GGA_STREAM
        return launch_status();
    }
    const Split sp = pick_split(m, k, n);
    if (!trans_a && trans_b && tall_abt(m, k, n)) {
        float* bt = static_cast<float*>(ws);  // b^T, [k][n]
        transpose_f32<<<dim3((unsigned)((k + 31) / 32), (unsigned)((n + 31) / 32)), 256, 0, s>>>(b, n, k, bt);
        b = bt;
        trans_b = 0;
    }
    GemmArgs g{};
    g.a = a;
    g.b = b;
    g.bias = bias;
    g.M = m;
    g.K = k;
    g.N = n;
    g.lda = trans_a ? m : k;
    g.ldb = trans_b ? k : n;
    g.trans_a = trans_a != 0;
    g.trans_b = trans_b != 0;
    g.kchunk = sp.kchunk;
    g.accumulate = accumulate;
    const int bn = pick_bn(n);
    const int64_t gy = (m + BM - 1) / BM, gx = (n + bn - 1) / bn;
    if (gy > 65535) return GGA_ERANGE;
    g.c = sp.splits > 1 ? static_cast<float*>(ws) : c;
    const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)sp.splits);
    if (bn == 64)
        gemm_f32_mfma<64><<<grid, kGemmThreads, 0, s>>>(g);
    else if (!g.trans_a && g.trans_b)
        gemm_f32_big<false, false><<<grid, kBigThreads, 0, s>>>(g);
    else if (!g.trans_a)
        gemm_f32_big<false, true><<<grid, kBigThreads, 0, s>>>(g);
    else if (g.trans_b)
        gemm_f32_big<true, false><<<grid, kBigThreads, 0, s>>>(g);
    else
        gemm_f32_big<true, true><<<grid, kBigThreads, 0, s>>>(g);
    if (sp.splits > 1) {
        const int64_t mn = (int64_t)m * n;
        splitk_reduce<<<(unsigned)((mn + 63) / 64), 1024, 0, s>>>(static_cast<const float*>(ws), sp.splits, mn, n,
                                                                bias, accumulate, c);
    }
    return launch_status();
}

}  // namespace

extern "C" int gga_linear(int32_t m, int32_t k, int32_t n, int32_t trans_a, int32_t trans_b, const float* a,
                          const float* b, const float* bias, float* c, void* ws, size_t ws_bytes, void* stream) {
    return linear_impl(m, k, n, trans_a, trans_b, a, b, bias, c, 0, ws, ws_bytes, stream);
}

extern "C" int gga_linear_accumulate(int32_t m, int32_t k, int32_t n, int32_t trans_a, int32_t trans_b,
                                     const float* a, const float* b, float* c, void* ws, size_t ws_bytes,
                                     void* stream) {
    return linear_impl(m, k, n, trans_a, trans_b, a, b, nullptr, c, 1, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- fused projections

namespace gga {
namespace {

// The fused products run on the 128 x 128 tile kernel without a k split.
bool fused_ok(int32_t m, int32_t k, int32_t n, int32_t seg, int32_t seg_mult) {
    return m >= 1 && seg >= 1 && seg % seg_mult == 0 && pick_split(m, k, n).splits == 1 && (m + BM - 1) / BM <= 65535;
}

}  // namespace
}  // namespace gga

extern "C" size_t gga_qkv_gate_proj_workspace(int32_t n, int32_t d) { return gga_linear_workspace(n, d, d); }

extern "C" int gga_qkv_gate_proj(int32_t n, int32_t d, const float* x, const float* w_q, const float* w_k,
                                 const float* w_v, const float* w_g, float b_g, float* q, float* k, float* v,
                                 float* gate_logit, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || d < 1) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!x || !w_q || !w_k || !w_v || !w_g || !q || !k || !v || !gate_logit) return GGA_EINVAL;
    if ((int64_t)n * d >= ((int64_t)1 << 40)) return GGA_ERANGE;
    hipStream_t s = as_stream(stream);
    bool aligned = true;
    for (const void* p : {(const void*)x, (const void*)w_q, (const void*)w_k, (const void*)w_v, (const void*)q,
                          (const void*)k, (const void*)v})
        aligned = aligned && aligned16(p);
    if (aligned && d % 4 == 0 && fused_ok(n, d, 3 * d, d, TT)) {
        // one product X [W_Q | W_K | W_V] over three column segments; column tile 0 also forms
        // the gate logit from the X rows it loads
        GemmArgs g{};
        g.a = x;
        g.b = w_q;
        g.c = q;
        g.M = n;
        g.K = d;
        g.N = 3 * d;
        g.lda = d;
        g.ldb = d;
        g.kchunk = d;
        g.nseg = 3;
        g.kseg = 1;
        g.seg_len = d;
        g.seg_b[0] = w_q;
        g.seg_b[1] = w_k;
        g.seg_b[2] = w_v;
        g.seg_c[0] = q;
        g.seg_c[1] = k;
        g.seg_c[2] = v;
        g.gate_w = w_g;
        g.gate_out = gate_logit;
        g.gate_b = b_g;
        const dim3 grid((unsigned)((3 * (int64_t)d) / TT), (unsigned)((n + BM - 1) / BM), 1);
        gemm_f32_seg_cols<<<grid, kBigThreads, 0, s>>>(g);
        return launch_status();
    }
    int st = gga_linear(n, d, d, 0, 0, x, w_q, nullptr, q, ws, ws_bytes, stream);
    if (st == GGA_OK) st = gga_linear(n, d, d, 0, 0, x, w_k, nullptr, k, ws, ws_bytes, stream);
    if (st == GGA_OK) st = gga_linear(n, d, d, 0, 0, x, w_v, nullptr, v, ws, ws_bytes, stream);
    if (st != GGA_OK) return st;
    gate_logit_kernel<<<(unsigned)(((int64_t)n + 3) / 4), 256, 0, s>>>(n, d, x, w_g, b_g, gate_logit);
    return launch_status();
}

extern "C" size_t gga_qkv_proj_bwd_x_workspace(int32_t n, int32_t d) {
    if (n < 0 || d < 1) return 0;
    const size_t wt = align_up((size_t)3 * d * d * sizeof(float), 256);
    const size_t lin = gga_linear_workspace(n, d, d);
    return wt > lin ? wt : lin;
}

extern "C" int gga_qkv_proj_bwd_x(int32_t n, int32_t d, const float* d_q, const float* d_k, const float* d_v,
                                  const float* w_q, const float* w_k, const float* w_v, const float* d_logit,
                                  const float* w_g, float* d_x, void* ws, size_t ws_bytes, void* stream) {
    if (n < 0 || d < 1) return GGA_EINVAL;
    if ((d_logit == nullptr) != (w_g == nullptr)) return GGA_EINVAL;
    if (n == 0) return GGA_OK;
    if (!d_q || !d_k || !d_v || !w_q || !w_k || !w_v || !d_x) return GGA_EINVAL;
    if ((int64_t)n * d >= ((int64_t)1 << 40)) return GGA_ERANGE;
    if (ws_bytes < gga_qkv_proj_bwd_x_workspace(n, d) || !ws) return GGA_EWORKSPACE;
    hipStream_t s = as_stream(stream);
    bool aligned = true;
    for (const void* p : {(const void*)d_q, (const void*)d_k, (const void*)d_v, (const void*)d_x, (const void*)ws})
        aligned = aligned && aligned16(p);
    if (aligned && d % 4 == 0 && fused_ok(n, 3 * d, d, d, TK2)) {
        // W^T of each projection into the workspace, then one product [dQ | dK | dV] [W_Q | W_K | W_V]^T
        // over three k segments, added into dX
        float* wt = static_cast<float*>(ws);
        const float* w[3] = {w_q, w_k, w_v};
        const dim3 tg((unsigned)((d + 31) / 32), (unsigned)((d + 31) / 32));
        for (int i = 0; i < 3; i++) transpose_f32<<<tg, 256, 0, s>>>(w[i], d, d, wt + (size_t)i * d * d);
        GemmArgs g{};
        g.a = d_q;
        g.b = wt;
        g.c = d_x;
        g.M = n;
        g.K = 3 * d;
        g.N = d;
        g.lda = d;
        g.ldb = d;
        g.kchunk = 3 * d;
        g.accumulate = 1;
        g.nseg = 1;
        g.kseg = 3;
        g.seg_len = d;
        g.seg_a[0] = d_q;
        g.seg_a[1] = d_k;
        g.seg_a[2] = d_v;
        for (int i = 0; i < 3; i++) g.seg_b[i] = wt + (size_t)i * d * d;
        g.r1_row = d_logit;  // + d_logit w_g^T in the same epilogue (null: none)
        g.r1_col = w_g;
        const dim3 grid((unsigned)((d + TT - 1) / TT), (unsigned)((n + BM - 1) / BM), 1);
        gemm_f32_seg_k<3><<<grid, kBigThreads, 0, s>>>(g);
        return launch_status();
    }
    int st = gga_linear_accumulate(n, d, d, 0, 1, d_q, w_q, d_x, ws, ws_bytes, stream);
    if (st == GGA_OK) st = gga_linear_accumulate(n, d, d, 0, 1, d_k, w_k, d_x, ws, ws_bytes, stream);
    if (st == GGA_OK) st = gga_linear_accumulate(n, d, d, 0, 1, d_v, w_v, d_x, ws, ws_bytes, stream);
    if (st == GGA_OK && d_logit) {
        const int64_t total = (int64_t)n * d;
        const int64_t blocks = (total + 255) / 256;
        rank1_add<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(n, d, d_logit, w_g, d_x);
        st = launch_status();
    }
    return st;
}
