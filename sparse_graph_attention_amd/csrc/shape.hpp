// Host-side choice of the lane layout of a node row and the checks of a local descriptor.
#pragma once

#include "common.hpp"

namespace gga {

struct Shape {
    int epl, hdp, ns, lpr_log2;
};

inline int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

inline int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) r++;
    return r;
}

// Picks the lane layout; returns false for shapes the kernels do not handle.
// Vector path: 16-byte element vectors when C is a multiple of 8 (bf16) or 4 (fp32);
// otherwise one element per lane.  At most two slots per lane on the vector path.
inline bool pick_shape(int H, int C, int dtype, Shape* sh) {
    const int vec = dtype == GGA_BF16 ? 8 : 4;
    sh->epl = (C % vec == 0) ? vec : 1;
    const int per_head = C / sh->epl;
    sh->hdp = next_pow2(per_head);
    if (sh->hdp > 64) return false;
    const int lanes = H * sh->hdp;
    if (lanes <= 64) {
        sh->ns = 1;
        sh->lpr_log2 = ilog2(next_pow2(lanes));
    } else {
        sh->ns = (lanes + 63) / 64;
        sh->lpr_log2 = 6;
        if (sh->ns > 2 || sh->epl == 1) return false;
    }
    return true;
}

// Rows of the source-side tensors (keys or source scores, values).
inline int32_t source_rows(const gga_local_desc* d) { return d->n_src > 0 ? d->n_src : d->n; }

inline int check_desc(const gga_local_desc* d) {
    if (!d) return GGA_EINVAL;
    if (d->n < 0 || d->e < 0 || d->heads < 1 || d->head_dim < 1 || d->n_src < 0) return GGA_EINVAL;
    if (d->e > (int64_t)INT32_MAX - 4096) return GGA_ERANGE;  // edge positions plus a loop stride fit int32
    const int64_t rows = d->n > source_rows(d) ? d->n : source_rows(d);
    if (rows * d->heads * d->head_dim >= ((int64_t)1 << 40)) return GGA_ERANGE;
    if (d->score != GGA_SCORE_DOT && d->score != GGA_SCORE_ADDITIVE && d->score != GGA_SCORE_MEAN)
        return GGA_EUNSUPPORTED;
    if (d->dtype != GGA_F32 && d->dtype != GGA_BF16) return GGA_EUNSUPPORTED;
    Shape sh;
    if (!pick_shape(d->heads, d->head_dim, d->dtype, &sh)) return GGA_EUNSUPPORTED;
    return GGA_OK;
}

}  // namespace gga
