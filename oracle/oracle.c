/*
 * Plain CPU oracle for neighbor-restricted multi-head graph attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code with the HIP library.
 *
 * Every routine is the plain definition written out: sequential loops, fp64
 * arithmetic on fp64 inputs, one destination row (or source row) at a time.
 * OpenMP splits the outer loop over rows only; each row's sums run in CSR order,
 * so results do not depend on the thread count.
 *
 * Edge direction (Tinymesh "Sparse attention experiment", section "Endpoint
 * projection"): an edge e: u -> v has source u and target v.  Sources provide
 * keys and values; targets provide queries and own the softmax group.
 *
 * Node tensors are [N, H, C] row-major; node scores are [N, H].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ROW(rows, i) ((rows) ? (int64_t)(rows)[i] : (int64_t)(i))

/*
 * Stable counting sort of a COO edge list by `key` (Tinymesh "Sparse attention
 * experiment", section "Target softmax": both segment reductions traverse the
 * destination CSR, and gathers return values in the original COO order).
 * key = dst gives the CSR by destination, key = src the CSR by source.
 * Within a row, edges keep ascending COO index.  Returns 0, or -1 if a key is out
 * of range (nothing is written then).
 */
int orc_coo_to_csr(int32_t n, int64_t e, const int32_t *key, const int32_t *other,
                   int32_t *row_ptr, int32_t *col, int32_t *eid) {
    for (int64_t i = 0; i < e; i++)
        if (key[i] < 0 || key[i] >= n) return -1;
    int64_t *cnt = (int64_t *)calloc((size_t)n + 1, sizeof(int64_t));
    for (int64_t i = 0; i < e; i++) cnt[key[i]]++;
    int64_t run = 0;
    for (int32_t v = 0; v < n; v++) {
        row_ptr[v] = (int32_t)run;
        int64_t c = cnt[v];
        cnt[v] = run; /* becomes the insertion cursor */
        run += c;
    }
    row_ptr[n] = (int32_t)run;
    for (int64_t i = 0; i < e; i++) {
        int64_t p = cnt[key[i]]++;
        col[p] = other[i];
        eid[p] = (int32_t)i;
    }
    free(cnt);
    return 0;
}

/*
 * Target softmax of one destination row's scores s[0..deg) (Tinymesh "Sparse
 * attention experiment", section "Target softmax"): alpha = exp(s - max) / sum.
 * Writes alpha into a[] and returns log-sum-exp = max + log(sum).
 */
static double row_softmax(const double *s, int64_t deg, double *a) {
    double m = -INFINITY;
    for (int64_t j = 0; j < deg; j++)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < deg; j++) {
        a[j] = exp(s[j] - m);
        z += a[j];
    }
    for (int64_t j = 0; j < deg; j++) a[j] /= z;
    return m + log(z);
}

/* Dot-product score of edge u -> v for head h ("Gated Local-Global Graph
 * Attention", Key formulas, local branch L_i: q_i k_j^T / sqrt(r)). */
static double dot_score(const double *q, const double *k, int64_t v, int64_t u, int h, int hh, int c,
                        double scale) {
    const double *qv = q + ((size_t)v * hh + h) * c;
    const double *ku = k + ((size_t)u * hh + h) * c;
    double s = 0.0;
    for (int i = 0; i < c; i++) s += qv[i] * ku[i];
    return s * scale;
}

/* GAT additive score: LeakyReLU(s_src[u] + s_dst[v]) (Tinymesh "Sparse attention
 * experiment", sections "Composition" and "Reference contract"). */
static double add_logit(const double *s_src, const double *s_dst, int64_t v, int64_t u, int h, int hh) {
    return s_src[(size_t)u * hh + h] + s_dst[(size_t)v * hh + h];
}
static double leaky(double z, double slope) { return z > 0.0 ? z : slope * z; }
static double leaky_grad(double z, double slope) { return z > 0.0 ? 1.0 : slope; }

/* Optional learned edge term of the additive logit (PyG GATConv with edge features, the
 * reference contract the Tinymesh page adopts; the page lists edge-feature scoring as not
 * yet covered): s_edge [E,H] in COO order, found through the CSR position's COO index. */
static double edge_term(const double *s_edge, const int32_t *eid, int64_t p, int h, int hh) {
    return s_edge ? s_edge[(size_t)eid[p] * hh + h] : 0.0;
}

/* Scores of all in-edges of v for head h, in CSR order. */
static void row_scores(int mode, const double *qs, const double *ks, int64_t v, int h, int hh, int c,
                       const int32_t *row_ptr, const int32_t *col, double scale, double slope,
                       const double *s_edge, const int32_t *eid, double *s) {
    int64_t b = row_ptr[v], e = row_ptr[v + 1];
    for (int64_t p = b; p < e; p++) {
        int64_t u = col[p];
        if (mode == 0) {
            s[p - b] = dot_score(qs, ks, v, u, h, hh, c, scale);
        } else {
            double zz = add_logit(ks, qs, v, u, h, hh) + edge_term(s_edge, eid, p, h, hh);
            s[p - b] = leaky(zz, slope);
        }
    }
}

/*
 * Local attention forward for destination rows `rows` (all N if rows == NULL):
 * out[v,h,:] = sum_e alpha_e * val[u,h,:], lse[v,h] = log sum_e exp(s_e).
 * mode 0: dot product, qs = q [N,H,C], ks = k [N,H,C].
 * mode 1: additive,    qs = s_dst [N,H], ks = s_src [N,H]; with s_edge (COO [E,H],
 *         NULL for none) and eid (the CSR's COO indices) the logit gains s_edge[e,h].
 * A row with no in-edges gets out = 0 and lse = -inf (isolated rows, Tinymesh
 * "Evidence and limits").  Heads are normalised independently and concatenated
 * (Tinymesh "Multiple heads are composition").
 */
void orc_local_fwd(int mode, int32_t n, int32_t hh, int32_t c, const double *qs, const double *ks,
                   const double *val, const int32_t *row_ptr, const int32_t *col, double scale, double slope,
                   const double *s_edge, const int32_t *eid, const int32_t *rows, int64_t n_rows, double *out,
                   double *lse) {
    (void)n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; i++) {
        int64_t v = ROW(rows, i);
        int64_t b = row_ptr[v], deg = row_ptr[v + 1] - b;
        double *s = (double *)malloc(sizeof(double) * (size_t)(deg > 0 ? deg : 1));
        double *a = (double *)malloc(sizeof(double) * (size_t)(deg > 0 ? deg : 1));
        for (int h = 0; h < hh; h++) {
            double *o = out + ((size_t)i * hh + h) * c;
            for (int j = 0; j < c; j++) o[j] = 0.0;
            if (deg == 0) {
                lse[(size_t)i * hh + h] = -INFINITY;
                continue;
            }
            row_scores(mode, qs, ks, v, h, hh, c, row_ptr, col, scale, slope, s_edge, eid, s);
            lse[(size_t)i * hh + h] = row_softmax(s, deg, a);
            for (int64_t p = 0; p < deg; p++) {
                const double *vu = val + ((size_t)col[b + p] * hh + h) * c;
                for (int j = 0; j < c; j++) o[j] += a[p] * vu[j];
            }
        }
        free(s);
        free(a);
    }
}

/*
 * Local attention backward, first-order gradients of the scalar sum(out * d_out).
 * Softmax gradient with the detached maximum (Tinymesh "Target softmax"): for
 * alpha = softmax(s) over a row, d s_e = alpha_e * (d alpha_e - sum_k alpha_k d alpha_k),
 * with d alpha_e = d_out[v] . val[u] per head.
 *
 * mode 0 (dot): dq[v] = sum_{e into v} ds_e * scale * k[u]
 *               dk[u] = sum_{e out of u} ds_e * scale * q[v]
 *               dval[u] = sum_{e out of u} alpha_e * d_out[v]
 * mode 1 (additive): dz_e = ds_e * LeakyReLU'(z_e);
 *               d_qs[v] (= d s_dst) = sum_{e into v} dz_e
 *               d_ks[u] (= d s_src) = sum_{e out of u} dz_e
 *               dval[u] = sum_{e out of u} alpha_e * d_out[v]
 * Sums "out of u" walk the CSR by source, grouping edge gradients by the
 * selected endpoint (Tinymesh "Endpoint projection", backward).
 *
 * With an edge term (mode 1, s_edge != NULL; eid / eid_s the COO indices of the CSR by
 * destination / by source), d_edge[e,h] = dz_e (COO order) for the edges into `rows_d`.
 *
 * Stage 1 computes, for every destination, lse and D = sum_e alpha_e d alpha_e
 * (written to lse_all / d_all, [N,H]).  Stage 2 fills d_qs for `rows_d`
 * (all if NULL), stage 3 fills d_ks and dval for `rows_s` (all if NULL);
 * outputs are indexed by position in those lists.
 */
void orc_local_bwd(int mode, int32_t n, int32_t hh, int32_t c, const double *qs, const double *ks,
                   const double *val, const double *d_out, const int32_t *row_ptr, const int32_t *col,
                   const int32_t *row_ptr_s, const int32_t *col_s, double scale, double slope,
                   const double *s_edge, const int32_t *eid, const int32_t *eid_s, double *d_edge,
                   double *lse_all, double *d_all, const int32_t *rows_d, int64_t n_rows_d, double *d_qs,
                   const int32_t *rows_s, int64_t n_rows_s, double *d_ks, double *d_val) {
    int qs_w = mode == 0 ? c : 1; /* width per head of qs / ks */

    /* stage 1: lse and D for every destination */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t v = 0; v < n; v++) {
        int64_t b = row_ptr[v], deg = row_ptr[v + 1] - b;
        double *s = (double *)malloc(sizeof(double) * (size_t)(deg > 0 ? deg : 1));
        double *a = (double *)malloc(sizeof(double) * (size_t)(deg > 0 ? deg : 1));
        for (int h = 0; h < hh; h++) {
            if (deg == 0) {
                lse_all[v * hh + h] = -INFINITY;
                d_all[v * hh + h] = 0.0;
                continue;
            }
            row_scores(mode, qs, ks, v, h, hh, c, row_ptr, col, scale, slope, s_edge, eid, s);
            lse_all[v * hh + h] = row_softmax(s, deg, a);
            const double *g = d_out + ((size_t)v * hh + h) * c;
            double dsum = 0.0;
            for (int64_t p = 0; p < deg; p++) {
                const double *vu = val + ((size_t)col[b + p] * hh + h) * c;
                double da = 0.0;
                for (int j = 0; j < c; j++) da += g[j] * vu[j];
                dsum += a[p] * da;
            }
            d_all[v * hh + h] = dsum;
        }
        free(s);
        free(a);
    }

    /* stage 2: gradient of the destination-side operand */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows_d; i++) {
        int64_t v = ROW(rows_d, i);
        int64_t b = row_ptr[v], e = row_ptr[v + 1];
        for (int h = 0; h < hh; h++) {
            double *dq = d_qs + ((size_t)i * hh + h) * qs_w;
            for (int j = 0; j < qs_w; j++) dq[j] = 0.0;
            if (e == b) continue;
            const double *g = d_out + ((size_t)v * hh + h) * c;
            double l = lse_all[v * hh + h], dd = d_all[v * hh + h];
            for (int64_t p = b; p < e; p++) {
                int64_t u = col[p];
                const double *vu = val + ((size_t)u * hh + h) * c;
                double da = 0.0;
                for (int j = 0; j < c; j++) da += g[j] * vu[j];
                if (mode == 0) {
                    double sc = dot_score(qs, ks, v, u, h, hh, c, scale);
                    double al = exp(sc - l);
                    double ds = al * (da - dd);
                    const double *ku = ks + ((size_t)u * hh + h) * c;
                    for (int j = 0; j < c; j++) dq[j] += ds * scale * ku[j];
                } else {
                    double z = add_logit(ks, qs, v, u, h, hh) + edge_term(s_edge, eid, p, h, hh);
                    double al = exp(leaky(z, slope) - l);
                    double ds = al * (da - dd);
                    dq[0] += ds * leaky_grad(z, slope);
                    if (d_edge) d_edge[(size_t)eid[p] * hh + h] = ds * leaky_grad(z, slope);
                }
            }
        }
    }

    /* stage 3: gradients of the source-side operands, over the CSR by source */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows_s; i++) {
        int64_t u = ROW(rows_s, i);
        int64_t b = row_ptr_s[u], e = row_ptr_s[u + 1];
        for (int h = 0; h < hh; h++) {
            double *dk = d_ks + ((size_t)i * hh + h) * qs_w;
            double *dv = d_val + ((size_t)i * hh + h) * c;
            for (int j = 0; j < qs_w; j++) dk[j] = 0.0;
            for (int j = 0; j < c; j++) dv[j] = 0.0;
            const double *vu = val + ((size_t)u * hh + h) * c;
            for (int64_t p = b; p < e; p++) {
                int64_t v = col_s[p];
                const double *g = d_out + ((size_t)v * hh + h) * c;
                double l = lse_all[v * hh + h], dd = d_all[v * hh + h];
                double da = 0.0;
                for (int j = 0; j < c; j++) da += g[j] * vu[j];
                double al;
                if (mode == 0) {
                    double sc = dot_score(qs, ks, v, u, h, hh, c, scale);
                    al = exp(sc - l);
                    double ds = al * (da - dd);
                    const double *qv = qs + ((size_t)v * hh + h) * c;
                    for (int j = 0; j < c; j++) dk[j] += ds * scale * qv[j];
                } else {
                    double z = add_logit(ks, qs, v, u, h, hh) + edge_term(s_edge, eid_s, p, h, hh);
                    al = exp(leaky(z, slope) - l);
                    double ds = al * (da - dd);
                    dk[0] += ds * leaky_grad(z, slope);
                }
                for (int j = 0; j < c; j++) dv[j] += al * g[j];
            }
        }
    }
}

/*
 * Endpoint projection (Tinymesh "Sparse attention experiment", section
 * "Endpoint projection"): out[e,:] = x[endpoint[e],:] for a node field [N,W].
 */
void orc_edge_values(int32_t w, const double *x, const int32_t *endpoint, int64_t e, double *out) {
    for (int64_t i = 0; i < e; i++)
        for (int j = 0; j < w; j++) out[(size_t)i * w + j] = x[(size_t)endpoint[i] * w + j];
}

/* Its backward: dx[u,:] = sum of d_edge[e,:] over edges whose selected endpoint is u,
 * taken as a row sum over the CSR keyed by that endpoint (row_ptr, eid). */
void orc_edge_values_bwd(int32_t n, int32_t w, const int32_t *row_ptr, const int32_t *eid, const double *d_edge,
                         double *dx) {
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t u = 0; u < n; u++) {
        for (int j = 0; j < w; j++) dx[(size_t)u * w + j] = 0.0;
        for (int64_t p = row_ptr[u]; p < row_ptr[u + 1]; p++)
            for (int j = 0; j < w; j++) dx[(size_t)u * w + j] += d_edge[(size_t)eid[p] * w + j];
    }
}

/*
 * A batch of graphs packed into one block-diagonal graph ("Gated Local-Global Graph
 * Attention", Implementation notes note 1: batched X with one adjacency list per graph).
 * Graph b owns nodes node_ptr[b] .. node_ptr[b+1]-1 and COO entries edge_ptr[b] ..
 * edge_ptr[b+1]-1 with local endpoint ids; each becomes id + node_ptr[b], or -1 when the
 * id is outside [0, n_b).  Returns the number of such endpoints.
 */
int64_t orc_batch_edges(int32_t b, const int32_t *node_ptr, const int32_t *edge_ptr, const int32_t *src_local,
                        const int32_t *dst_local, int32_t *src, int32_t *dst) {
    int64_t bad = 0;
    for (int32_t g = 0; g < b; g++) {
        const int32_t nb = node_ptr[g + 1] - node_ptr[g];
        for (int64_t i = edge_ptr[g]; i < edge_ptr[g + 1]; i++) {
            const int32_t s = src_local[i], d = dst_local[i];
            src[i] = (s >= 0 && s < nb) ? s + node_ptr[g] : -1;
            dst[i] = (d >= 0 && d < nb) ? d + node_ptr[g] : -1;
            bad += (src[i] < 0) + (dst[i] < 0);
        }
    }
    return bad;
}

/*
 * Relation-typed messages (GiGL pull request "Support relation message modes on the
 * packed GraphTransformerEncoder path", section "Approach": per-relation transforms,
 * mean or softmax weighting, scatter-add into the targets).  Edge e: u -> v of relation
 * r carries the message val_r[u] = x_u W_V^r; in softmax mode its score for head h is
 * scale * q[v,h] . key_r[u,h] with key_r[u] = x_u W_K^r.  The weights of v's in-edges
 * (all relations together) are the target softmax of those scores (softmax mode) or
 * 1/deg(v) each (mean mode); out[v] = sum of weight * message.
 *
 * Per-relation tensors are [R, N, H, C]; rel is the relation of each COO edge and eid
 * the COO index of each CSR position, so the relation of CSR position p is rel[eid[p]].
 * mode 0: softmax (q, key needed); mode 1: mean (q, key unused, may be NULL).
 * lse[v,h] is the log of the softmax normaliser (log deg(v) in mean mode); a row with
 * no in-edges gets out = 0 and lse = -inf.
 */
static const double *rel_row(const double *t, int32_t n, int32_t hh, int32_t c, int32_t r, int64_t u, int h) {
    return t + ((((size_t)r * n + (size_t)u) * hh + h) * c);
}

static void relation_weights(int mode, int32_t n, int32_t hh, int32_t c, const double *q, const double *key,
                             int64_t v, int h, const int32_t *row_ptr, const int32_t *col, const int32_t *rel,
                             const int32_t *eid, double scale, double *s, double *a, double *lse) {
    const int64_t b = row_ptr[v], deg = row_ptr[v + 1] - b;
    if (deg == 0) {
        *lse = -INFINITY;
        return;
    }
    if (mode == 1) {
        for (int64_t j = 0; j < deg; j++) a[j] = 1.0 / (double)deg;
        *lse = log((double)deg);
        return;
    }
    const double *qv = q + ((size_t)v * hh + h) * c;
    for (int64_t j = 0; j < deg; j++) {
        const double *k = rel_row(key, n, hh, c, rel[eid[b + j]], col[b + j], h);
        double d = 0.0;
        for (int i = 0; i < c; i++) d += qv[i] * k[i];
        s[j] = d * scale;
    }
    *lse = row_softmax(s, deg, a);
}

void orc_relation_fwd(int mode, int32_t n, int32_t hh, int32_t c, const double *q, const double *key,
                      const double *val, const int32_t *row_ptr, const int32_t *col, const int32_t *rel,
                      const int32_t *eid, double scale, const int32_t *rows, int64_t n_rows, double *out,
                      double *lse) {
    int64_t maxdeg = 0;
    for (int64_t v = 0; v < n; v++)
        if (row_ptr[v + 1] - row_ptr[v] > maxdeg) maxdeg = row_ptr[v + 1] - row_ptr[v];
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(maxdeg + 1));
        double *a = (double *)malloc(sizeof(double) * (size_t)(maxdeg + 1));
#pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < n_rows; i++) {
            const int64_t v = ROW(rows, i);
            const int64_t b = row_ptr[v], deg = row_ptr[v + 1] - b;
            for (int h = 0; h < hh; h++) {
                double *o = out + ((size_t)i * hh + h) * c;
                for (int x = 0; x < c; x++) o[x] = 0.0;
                relation_weights(mode, n, hh, c, q, key, v, h, row_ptr, col, rel, eid, scale, s, a,
                                 &lse[(size_t)i * hh + h]);
                for (int64_t j = 0; j < deg; j++) {
                    const double *m = rel_row(val, n, hh, c, rel[eid[b + j]], col[b + j], h);
                    for (int x = 0; x < c; x++) o[x] += a[j] * m[x];
                }
            }
        }
        free(s);
        free(a);
    }
}

/*
 * First-order gradients of sum(out * d_out) for orc_relation_fwd over all rows.  Per edge
 * e (target v, source u, relation r) and head h, with weight a_e, da_e = d_out[v] . val_r[u]
 * and D_v = d_out[v] . out[v]:
 *   d_val_r[u]  += a_e d_out[v]
 *   softmax mode, ds_e = a_e (da_e - D_v):  d_q[v] += scale ds_e key_r[u],
 *                                            d_key_r[u] += scale ds_e q[v]
 * The mean weights do not depend on the inputs.  Rows are visited in order and each
 * head's sums touch that head's slice only, so the result does not depend on the thread
 * count.  d_q and d_key may be NULL in mean mode.
 */
void orc_relation_bwd(int mode, int32_t n, int32_t n_rel, int32_t hh, int32_t c, const double *q,
                      const double *key, const double *val, const double *d_out, const int32_t *row_ptr,
                      const int32_t *col, const int32_t *rel, const int32_t *eid, double scale, double *d_q,
                      double *d_key, double *d_val) {
    const size_t rel_size = (size_t)n_rel * n * hh * c;
    memset(d_val, 0, sizeof(double) * rel_size);
    if (mode == 0) {
        memset(d_key, 0, sizeof(double) * rel_size);
        memset(d_q, 0, sizeof(double) * (size_t)n * hh * c);
    }
    int64_t maxdeg = 0;
    for (int64_t v = 0; v < n; v++)
        if (row_ptr[v + 1] - row_ptr[v] > maxdeg) maxdeg = row_ptr[v + 1] - row_ptr[v];
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(maxdeg + 1));
        double *a = (double *)malloc(sizeof(double) * (size_t)(maxdeg + 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)c);
#pragma omp for schedule(static, 1)
        for (int h = 0; h < hh; h++) {
            for (int64_t v = 0; v < n; v++) {
                const int64_t b = row_ptr[v], deg = row_ptr[v + 1] - b;
                if (deg == 0) continue;
                double lse;
                relation_weights(mode, n, hh, c, q, key, v, h, row_ptr, col, rel, eid, scale, s, a, &lse);
                const double *g = d_out + ((size_t)v * hh + h) * c;
                for (int x = 0; x < c; x++) o[x] = 0.0;
                for (int64_t j = 0; j < deg; j++) {
                    const double *m = rel_row(val, n, hh, c, rel[eid[b + j]], col[b + j], h);
                    for (int x = 0; x < c; x++) o[x] += a[j] * m[x];
                }
                double dd = 0.0;
                for (int x = 0; x < c; x++) dd += g[x] * o[x];
                const double *qv = mode == 0 ? q + ((size_t)v * hh + h) * c : NULL;
                double *dq = mode == 0 ? d_q + ((size_t)v * hh + h) * c : NULL;
                for (int64_t j = 0; j < deg; j++) {
                    const int32_t r = rel[eid[b + j]];
                    const int64_t u = col[b + j];
                    const double *m = rel_row(val, n, hh, c, r, u, h);
                    double *dm = d_val + (rel_row(val, n, hh, c, r, u, h) - val);
                    for (int x = 0; x < c; x++) dm[x] += a[j] * g[x];
                    if (mode != 0) continue;
                    double da = 0.0;
                    for (int x = 0; x < c; x++) da += g[x] * m[x];
                    const double ds = a[j] * (da - dd) * scale;
                    const double *k = rel_row(key, n, hh, c, r, u, h);
                    double *dk = d_key + (k - key);
                    for (int x = 0; x < c; x++) {
                        dq[x] += ds * k[x];
                        dk[x] += ds * qv[x];
                    }
                }
            }
        }
        free(s);
        free(a);
        free(o);
    }
}

/* Thread count of the OpenMP loops (benchmark baselines time one thread and all). */
void orc_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
