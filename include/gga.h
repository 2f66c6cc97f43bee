/*
 * gga.h -- C ABI of libgga, neighbor-restricted multi-head graph attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Graph.  A directed multigraph on n nodes given as a COO edge list of int32
 *   (src[e], dst[e]).  Edge e: u -> v has source u and target v (Tinymesh
 *   "Sparse attention experiment", section "Endpoint projection").  The source
 *   provides keys and values, the target provides the query and owns the
 *   softmax group (the in-edges of v).  Self-loops are ordinary edges that the
 *   caller adds; the library never adds, removes, deduplicates or reorders
 *   edges (section "Composition": no silent topology change).  Duplicate edges
 *   each contribute their own softmax term.
 * CSR.  row_ptr[n+1], col[E], eid[E] as built by gga_coo_to_csr: row v holds
 *   the edges whose key is v, in ascending COO index; eid is that COO index and
 *   col the other endpoint.
 * Node tensors.  Row-major [n, H, C] with heads as contiguous chunks of the
 *   feature axis ("ag_multihead_attention", Details: head h is rows
 *   h*d_k .. (h+1)*d_k-1); node scores are [n, H].  Outputs are fp32.
 * Memory.  Every pointer is a device pointer owned by the caller.  The library
 *   never allocates, frees or retains device memory; scratch comes from a
 *   caller buffer `ws` of at least the size the matching *_workspace query
 *   returns (a NULL ws is allowed when that size is 0).  Inputs are never
 *   written.  Pointers to node tensors must be 16-byte aligned.
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues work on it: no call synchronises or copies device -> host.
 * Errors.  Arguments are checked on the host before anything is enqueued; on a
 *   failed check the call returns a nonzero status and enqueues nothing.  Edge
 *   index ranges are not checked by the compute calls (they would need a device
 *   read): run gga_validate_coo on untrusted input first.  A HIP launch error is
 *   returned as GGA_EHIP.  n == 0 or E == 0 are valid and return GGA_OK.
 * Threads.  Calls are re-entrant; the library keeps no mutable global state,
 *   except the fixed scratch array of gga_local_attn_fwd_noalloc (see there).
 */
#ifndef GGA_H
#define GGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GGA_ABI_VERSION 4

/* status codes */
#define GGA_OK 0
#define GGA_EINVAL 1       /* null pointer with a nonzero size, negative size, misalignment */
#define GGA_ERANGE 2       /* a size beyond what int32 indexing supports */
#define GGA_EUNSUPPORTED 3 /* dtype, score mode or shape the library does not handle */
#define GGA_EWORKSPACE 4   /* workspace or plan buffer smaller than its query says */
#define GGA_EHIP 5         /* a HIP runtime call or kernel launch failed */
#define GGA_ESCRATCH 6     /* gga_local_attn_fwd_noalloc: the input needs more than its fixed scratch */

/* storage type of node tensors */
#define GGA_F32 0
#define GGA_BF16 1

/* score of edge u -> v */
#define GGA_SCORE_DOT 0      /* scale * q[v,h,:] . k[u,h,:] */
#define GGA_SCORE_ADDITIVE 1 /* LeakyReLU(s_src[u,h] + s_dst[v,h]) */
#define GGA_SCORE_MEAN 2     /* no score: every in-edge of v weighs 1/deg(v) */

int gga_abi_version(void);
const char *gga_status_string(int status);

/*
 * Count COO entries whose src or dst lies outside [0, n).  Writes the count to the
 * device int *d_bad (the call clears it first).  The only check of index range.
 */
int gga_validate_coo(int32_t n, int64_t e, const int32_t *src, const int32_t *dst, int32_t *d_bad, void *stream);

/*
 * COO -> CSR by `key` with a stable counting sort (Tinymesh "Sparse attention
 * experiment", section "Target softmax": the segment reductions traverse the
 * destination CSR and gathers keep the original COO order).
 *   key = dst, other = src: the CSR by destination used by the forward pass.
 *   key = src, other = dst: the CSR by source used by the backward pass.
 * Outputs row_ptr[n+1], col[e] (= other[eid]) and eid[e]; within a row eid
 * ascends.  The result is a pure function of the input (bit-exact, no
 * dependence on scheduling).  Keys outside [0, n) are skipped in the row
 * counts; the outputs are then unspecified but every write stays in bounds.
 * e must be < 2^31.
 */
size_t gga_coo_to_csr_workspace(int32_t n, int64_t e);
int gga_coo_to_csr(int32_t n, int64_t e, const int32_t *key, const int32_t *other, int32_t *row_ptr, int32_t *col,
                   int32_t *eid, void *ws, size_t ws_bytes, void *stream);

/*
 * Degree-bucket plan of a CSR, built once per fixed topology.  Rows with few
 * edges are processed by one wavefront each; longer rows by a workgroup; rows
 * longer than one chunk are split into chunks whose partial softmax states are
 * merged in a fixed order, so that high-degree rows do not serialise (Tinymesh
 * "Sparse attention experiment", section "Target softmax", which notes that
 * high-degree rows serialise in a plain pull kernel).  The plan is an opaque
 * device buffer of gga_plan_bytes(n, e) bytes; it depends only on row_ptr.
 */
size_t gga_plan_bytes(int32_t n, int64_t e);
size_t gga_plan_workspace(int32_t n, int64_t e);
int gga_plan_build(int32_t n, int64_t e, const int32_t *row_ptr, void *plan, size_t plan_bytes, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * The plan records the n and e it was built for.  No topology is changed behind
 * the caller's back (Tinymesh "Sparse attention experiment", section "Reference
 * contract"): a row of row_ptr outside [0, e] (or rows that together overflow the
 * tables sized for e edges) marks the plan invalid at build time, and a kernel
 * handed a plan built for another n or e, or an invalid one, processes no row and
 * writes nothing (its outputs keep their contents) and marks the plan as misused.
 * gga_plan_status writes to the device int *d_status, in stream order: GGA_OK,
 * GGA_ERANGE (row_ptr inconsistent with e) or GGA_EINVAL (not a plan for this n
 * and e, or misused by an earlier call).  The caller reads it when it chooses.
 */
int gga_plan_status(const void *plan, int32_t n, int64_t e, int32_t *d_status, void *stream);

/* Shape and mode of a local attention call. */
typedef struct gga_local_desc {
    int32_t n;            /* nodes */
    int32_t heads;        /* H */
    int64_t e;            /* edges (length of col), at most 2^31 - 4097 (GGA_ERANGE) */
    int32_t head_dim;     /* C (r): per-head width */
    int32_t score;        /* GGA_SCORE_DOT, GGA_SCORE_ADDITIVE or GGA_SCORE_MEAN */
    int32_t dtype;        /* storage type of q, k, v (dot) or of v (additive, mean) */
    float scale;          /* dot: multiplier of q.k, usually 1/sqrt(C) */
    float negative_slope; /* additive: LeakyReLU slope, usually 0.2 */
    int32_t n_src;        /* rows of the source-side tensors (ks, v); 0 means n */
} gga_local_desc;

/*
 * Shapes the local kernels handle (others give GGA_EUNSUPPORTED before any
 * launch).  A head's C values are read E at a time, E = 8 for bf16 with C a
 * multiple of 8, 4 for fp32 with C a multiple of 4, else 1; a head takes
 * P = next power of two >= C / E lanes, and P <= 64.  With E > 1 the H heads
 * take at most two wavefront slots (H * P <= 128: bf16 up to C = 512 for one
 * head or H * C <= 1024; fp32 up to C = 256 or H * C <= 512); with E = 1 they
 * take one (H * P <= 64).
 */

/*
 * Local attention forward ("Gated Local-Global Graph Attention", Key formulas,
 * local branch L_i; Tinymesh "Sparse attention experiment", sections
 * "Composition", "Multiple heads are composition" and "Target softmax").
 * For every target v and head h, over the in-edges e: u -> v of the CSR by
 * destination:
 *   dot:      s_e = scale * q[v,h,:] . k[u,h,:]      (qs = q, ks = k: [n,H,C])
 *   additive: s_e = LeakyReLU(s_src[u,h] + s_dst[v,h]) (qs = s_dst, ks = s_src:
 *             fp32 [n,H])
 *   mean:     s_e = 0, so alpha_e = 1/deg(v)         (qs, ks unused, may be NULL;
 *             GiGL pull request "Support relation message modes on the packed
 *             GraphTransformerEncoder path", section "Approach": mean weighting)
 *   alpha_e = exp(s_e - max) / sum exp(s - max)       (per v, h)
 *   out[v,h,:] = sum_e alpha_e v[u,h,:]               (fp32 [n,H,C])
 *   lse[v,h] = log sum_e exp(s_e)                     (fp32 [n,H]; may be NULL)
 * A row with no in-edges gets out = 0 and lse = -inf.  Heads are normalised
 * independently and concatenated.  `plan` comes from gga_plan_build on the same
 * row_ptr.  Deterministic: the same inputs give bit-identical outputs.
 * Sources and targets may index different row sets: with d->n_src > 0 the
 * source-side tensors (k or s_src, and v) have n_src rows and col holds ids in
 * [0, n_src), e.g. one row per (node, relation) pair (gga_relation_sources).
 */
size_t gga_local_attn_fwd_workspace(const gga_local_desc *d);
int gga_local_attn_fwd(const gga_local_desc *d, const void *qs, const void *ks, const void *v,
                       const int32_t *row_ptr, const int32_t *col, const void *plan, float *out, float *lse,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Allocation-free local attention forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and bits as gga_local_attn_fwd, with the
 * partial softmax states of split rows kept in a fixed device array of 96 MiB that the
 * library holds on each device it runs on until the process ends, instead of a caller
 * workspace.  Nothing is allocated or freed; the caller passes inputs and outputs.
 * Inputs whose gga_local_attn_fwd_workspace(d) exceeds 96 MiB are rejected with
 * GGA_ESCRATCH before anything is enqueued (with rows of H*C = 512 values that allows
 * about 24M edges, with 256 values about 47M).  The stream must belong to the current
 * device.  Every call on a device shares that device's array, and nothing in it needs
 * to start cleared: calls that overlap in time on one device (different streams, or
 * different host threads) race on it and must be serialised by the caller.
 */
int gga_local_attn_fwd_noalloc(const gga_local_desc *d, const void *qs, const void *ks, const void *v,
                               const int32_t *row_ptr, const int32_t *col, const void *plan, float *out,
                               float *lse, void *stream);

/*
 * Local attention backward: first-order gradients of sum(out * d_out), with the
 * softmax maximum treated as a constant (Tinymesh "Sparse attention experiment",
 * section "Target softmax").  With d_alpha_e = d_out[v,h,:] . v[u,h,:],
 * D[v,h] = sum_e alpha_e d_alpha_e and ds_e = alpha_e (d_alpha_e - D[v,h]):
 *   dot:      d_qs = dq[v] = sum_{e into v} ds_e scale k[u]          fp32 [n,H,C]
 *             d_ks = dk[u] = sum_{e out of u} ds_e scale q[v]        fp32 [n,H,C]
 *   additive: d_qs = d s_dst[v] = sum_{e into v} ds_e LeakyReLU'(z_e) fp32 [n,H]
 *             d_ks = d s_src[u] = sum_{e out of u} ds_e LeakyReLU'(z_e)
 *   all:      d_v[u] = sum_{e out of u} alpha_e d_out[v]              fp32 [n,H,C]
 * Sums over the edges out of u walk the CSR by source (row_ptr_s, col_s with
 * plan_s), grouping edge gradients by the selected endpoint (section "Endpoint
 * projection", backward), so no floating-point atomics are used and results are
 * deterministic.  `out` and `lse` are the forward's outputs.
 * Mean mode has constant weights 1/deg(v) (taken from row_ptr): only d_v is
 * written; qs, ks, out, lse, d_qs and d_ks are unused and may be NULL.
 * With d->n_src > 0, d_ks and d_v have n_src rows and the CSR by source (row_ptr_s
 * with n_src + 1 entries, plan_s built for n_src rows) is keyed by source ids in
 * [0, n_src).
 */
size_t gga_local_attn_bwd_workspace(const gga_local_desc *d);
int gga_local_attn_bwd(const gga_local_desc *d, const void *qs, const void *ks, const void *v, const float *out,
                       const float *lse, const float *d_out, const int32_t *row_ptr, const int32_t *col,
                       const void *plan, const int32_t *row_ptr_s, const int32_t *col_s, const void *plan_s,
                       float *d_qs, float *d_ks, float *d_v, void *ws, size_t ws_bytes, void *stream);

/*
 * Relation-typed edges (GiGL pull request "Support relation message modes on the
 * packed GraphTransformerEncoder path", section "Approach": relation edges travel as
 * packed rows (target, source, relation) with host-side (relation, start, end)
 * segments, and messages go through per-relation transforms).  Maps each edge to the
 * row of a per-relation node tensor: projecting all n nodes by the R transforms side
 * by side gives [n, R*W], which viewed as [n*R, W] holds node u under relation r in
 * row u*R + r.  So
 *   src_rel[i] = src[i] * R + r   for the segment (r, start, end) with start <= i < end
 * and the local attention calls run with d->n_src = n*R over (src_rel, dst).
 * seg is HOST memory: n_seg triples (relation, start, end) of int32, in order, each
 * starting where the previous ended (the first at 0, the last ending at e), possibly
 * empty, with relation in [0, R); anything else returns GGA_EINVAL.  A src outside
 * [0, n) is written as -1 and a dst outside [0, n) is left as it is; both are counted
 * in the device int *d_bad (cleared first): run no compute call on a nonzero count.
 * n * R must be < 2^31 (GGA_ERANGE).  Bit-exact.
 */
int gga_relation_sources(int32_t n, int32_t relations, int64_t e, const int32_t *src, const int32_t *dst,
                         int32_t n_seg, const int32_t *seg, int32_t *src_rel, int32_t *d_bad, void *stream);

/*
 * Endpoint projection (Tinymesh "Sparse attention experiment", section
 * "Endpoint projection"): out[e,:] = x[endpoint[e],:] for a node field x of
 * [n, width] elements of `dtype`; out is [e, width] of the same dtype.  Pass
 * endpoint = src for "source", dst for "target".
 */
int gga_edge_values(int32_t n, int32_t width, int32_t dtype, const void *x, int64_t e, const int32_t *endpoint,
                    void *out, void *stream);

/*
 * Its backward: dx[u,:] = sum of d_edge[e,:] over the edges whose selected
 * endpoint is u, as a row sum over the CSR keyed by that endpoint (row_ptr, eid
 * from gga_coo_to_csr with key = endpoint).  fp32, deterministic.
 */
int gga_edge_values_bwd(int32_t n, int32_t width, int64_t e, const int32_t *row_ptr, const int32_t *eid,
                        const float *d_edge, float *dx, void *stream);

/*
 * GAT node coefficients (Tinymesh "Sparse attention experiment", section
 * "Composition": one source and one target coefficient per node and head):
 *   s_src[n,h] = sum_c a_s[h,c] hf[n,h,c],  s_dst[n,h] = sum_c a_t[h,c] hf[n,h,c]
 * hf fp32 [n,H,C]; a_s, a_t fp32 [H,C]; outputs fp32 [n,H].  a_t and s_dst may both
 * be NULL (one coefficient per row, e.g. the edge term a_e . HE over edge rows).
 */
int gga_gat_coef_fwd(int32_t n, int32_t heads, int32_t head_dim, const float *hf, const float *a_s,
                     const float *a_t, float *s_src, float *s_dst, void *stream);

/*
 * Backward of the coefficients, joined with the aggregation gradient d_hf_attn
 * from gga_local_attn_bwd (additive mode):
 *   d_hf[n,h,c] = d_hf_attn[n,h,c] + a_s[h,c] d_s_src[n,h] + a_t[h,c] d_s_dst[n,h]
 *   d_a_s[h,c] = sum_n d_s_src[n,h] hf[n,h,c],  d_a_t likewise with d_s_dst.
 * The sums over n use a fixed two-level order (deterministic).  d_hf may alias
 * d_hf_attn.  d_hf_attn may be NULL (zero); a_t, d_s_dst and d_a_t may all be NULL
 * (one coefficient per row).
 */
size_t gga_gat_coef_bwd_workspace(int32_t n, int32_t heads, int32_t head_dim);
int gga_gat_coef_bwd(int32_t n, int32_t heads, int32_t head_dim, const float *hf, const float *a_s,
                     const float *a_t, const float *d_hf_attn, const float *d_s_src, const float *d_s_dst,
                     float *d_hf, float *d_a_s, float *d_a_t, void *ws, size_t ws_bytes, void *stream);

/*
 * Dense fp32 product on the matrix cores: c[m,n] = op(a) op(b) (+ bias[n]),
 * op(a) = a [m,k] or, with trans_a, a stored [k,m]; op(b) = b [k,n] or, with
 * trans_b, b stored [n,k].  Row-major, fp32 in and out, fp32 accumulation.
 * Used for the projections Q = X W_Q, K, V, the output map W_o, the GAT map
 * X W and its gradients X^T dH, dH W^T ("Gated Local-Global Graph Attention",
 * Mathematical statement; Tinymesh "Composition").  bias may be NULL.  When
 * the output is small and k long, k is split into a fixed number of ranges
 * whose partial products (in `ws`) are added in range order: deterministic.
 * For a tall a times a small b stored [n,k] (trans_b), b is first transposed
 * into `ws` (same results).  gga_linear_workspace does not know the transposes
 * and returns enough for either use.
 */
size_t gga_linear_workspace(int32_t m, int32_t k, int32_t n);
int gga_linear(int32_t m, int32_t k, int32_t n, int32_t trans_a, int32_t trans_b, const float *a, const float *b,
               const float *bias, float *c, void *ws, size_t ws_bytes, void *stream);

/*
 * Global linear-attention branch ("Gated Local-Global Graph Attention", Key
 * formulas G_i, S, z; Implementation notes item 2: phi = elu + 1), per head h:
 *   S[h] = sum_j phi(k[j,h,:]) v[j,h,:]^T   fp32 [H,r,r]
 *   z[h] = sum_j phi(k[j,h,:])              fp32 [H,r]
 *   g[i,h,:] = phi(q[i,h,:])^T S[h] / (phi(q[i,h,:]) . z[h] + eps)   fp32 [n,H,r]
 * q, k, v fp32 [n,H,r].  The sums over j use a fixed split order
 * (deterministic).  s_out and z_out may be NULL.
 */
size_t gga_global_linear_workspace(int32_t n, int32_t heads, int32_t r);
int gga_global_linear_fwd(int32_t n, int32_t heads, int32_t r, const float *q, const float *k, const float *v,
                          float eps, float *s_out, float *z_out, float *g_out, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * The layer's projections in one product ("Gated Local-Global Graph Attention",
 * Mathematical statement: Q = X W_Q, K = X W_K, V = X W_V; Key formulas: the node gate
 * g_i = sigmoid(x_i . w_g + b_g)):
 *   [Q | K | V | gate_logit] = X [W_Q | W_K | W_V | w_g] + [0 | 0 | 0 | b_g]
 * x fp32 [n,d]; w_q, w_k, w_v fp32 [d,d]; w_g fp32 [d]; q, k, v fp32 [n,d] (each its own
 * tensor, viewed [n,H,d/H] by the attention calls); gate_logit fp32 [n] (before the
 * sigmoid).  With d a multiple of 128 and 16-byte aligned rows this is one launch on the
 * matrix cores that reads X once, the gate logit formed from the X rows the first column
 * tile loads; otherwise three gga_linear products and a row kernel (same results up to
 * fp32 summation order).  Workspace: gga_qkv_gate_proj_workspace (for the second path).
 */
size_t gga_qkv_gate_proj_workspace(int32_t n, int32_t d);
int gga_qkv_gate_proj(int32_t n, int32_t d, const float *x, const float *w_q, const float *w_k, const float *w_v,
                      const float *w_g, float b_g, float *q, float *k, float *v, float *gate_logit, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * Node gate and combination ("Gated Local-Global Graph Attention", Key formulas):
 *   gate[i] = sigmoid(gate_logit[i])                 (gate_logit fp32 [n], from
 *                                                     gga_qkv_gate_proj: x_i . w_g + b_g)
 *   y[i,:] = gate[i] l[i,:] + (1 - gate[i]) g[i,:]   (l, g, y fp32 [n,width])
 * gate_out may be NULL.
 */
int gga_gated_combine(int32_t n, int32_t width, const float *gate_logit, const float *l, const float *g,
                      float *gate_out, float *y, void *stream);

/*
 * Residual and LayerNorm of the layer output ("Gated Local-Global Graph
 * Attention", Implementation notes item 2: LayerNorm(X + Wo(...))):
 *   a = x + y;  out = gamma (a - mean(a)) / sqrt(var(a) + eps) + beta
 * over the last axis of width d, biased variance; all fp32 [n,d], gamma/beta [d].
 */
int gga_add_layernorm(int32_t n, int32_t d, const float *x, const float *y, const float *gamma, const float *beta,
                      float eps, float *out, void *stream);

/* ------------------------------------------------------------------------
 * Backward of the gated local-global layer ("Gated Local-Global Graph
 * Attention", Implementation notes item 2), first-order gradients of
 * sum(out * d_out).  The local branch's gradient is gga_local_attn_bwd.
 * ------------------------------------------------------------------------ */

/*
 * c[m,n] += op(a) op(b): gga_linear accumulating into c instead of overwriting it
 * (same shapes, layouts, workspace and determinism).  Used to add the projection
 * gradients dQ W_Q^T, dK W_K^T, dV W_V^T into dX.
 */
int gga_linear_accumulate(int32_t m, int32_t k, int32_t n, int32_t trans_a, int32_t trans_b, const float *a,
                          const float *b, float *c, void *ws, size_t ws_bytes, void *stream);

/*
 * The input gradient of the three projections (and of the gate logit) in one product:
 *   d_x += [d_q | d_k | d_v] [W_Q | W_K | W_V]^T (+ d_logit w_g^T)
 *        = d_q W_Q^T + d_k W_K^T + d_v W_V^T (+ d_logit w_g^T)
 * d_q, d_k, d_v fp32 [n,d]; w_q, w_k, w_v fp32 [d,d]; d_x fp32 [n,d], added to.  d_logit
 * fp32 [n] and w_g fp32 [d] are both given or both NULL: the gate logit's share of the input
 * gradient (gga_gated_combine_bwd's d_logit), added in the same epilogue.  With d % 4 == 0
 * and 16-byte aligned rows, one accumulating launch (the three W^T staged in the workspace,
 * the k ranges taken in the order q, k, v); otherwise three gga_linear_accumulate calls in
 * that order, then the d_logit term.  Workspace: gga_qkv_proj_bwd_x_workspace.
 */
size_t gga_qkv_proj_bwd_x_workspace(int32_t n, int32_t d);
int gga_qkv_proj_bwd_x(int32_t n, int32_t d, const float *d_q, const float *d_k, const float *d_v, const float *w_q,
                       const float *w_k, const float *w_v, const float *d_logit, const float *w_g, float *d_x,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of out = LayerNorm(x + y) over rows of width d (gga_add_layernorm):
 *   d_pre[i,:] = rstd (g - mean(g) - xhat mean(g xhat)),  g = d_out gamma,
 *   d_gamma = sum_i d_out xhat,  d_beta = sum_i d_out
 * with xhat and rstd recomputed from x + y.  d_pre is the gradient of x + y (so of both
 * x and y).  The sums over rows use a fixed two-level order (deterministic).  fp32.
 */
size_t gga_add_layernorm_bwd_workspace(int32_t n, int32_t d);
int gga_add_layernorm_bwd(int32_t n, int32_t d, const float *x, const float *y, const float *gamma, float eps,
                          const float *d_out, float *d_pre, float *d_gamma, float *d_beta, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Backward of the gate and combination (gga_gated_combine), with g_i recomputed:
 *   d_l = g dY,  d_g = (1 - g) dY,  dt_i = g_i (1 - g_i) sum_c dY[i,c] (l[i,c] - g[i,c])
 *   d_x_out = d_x_in + dt w_g^T   (d_x_out may alias d_x_in)
 *   d_logit = dt                  (fp32 [n], may be NULL)
 *   d_w_g = sum_i dt_i x_i,  d_b_g = sum_i dt_i   (fixed two-level order)
 * x [n,d]; l, g_glob, d_y, d_l, d_g [n,width]; d_w_g [d]; d_b_g one float.  d_x_in and
 * d_x_out are both given or both NULL; with both NULL, d_logit must be given and the caller
 * adds dt w_g^T into its input gradient elsewhere (gga_qkv_proj_bwd_x takes d_logit), which
 * saves reading and writing an [n,d] gradient here.
 */
size_t gga_gated_combine_bwd_workspace(int32_t n, int32_t d);
int gga_gated_combine_bwd(int32_t n, int32_t d, const float *x, const float *w_g, float b_g, int32_t width,
                          const float *l, const float *g_glob, const float *d_y, float *d_l, float *d_g,
                          const float *d_x_in, float *d_x_out, float *d_logit, float *d_w_g, float *d_b_g,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of the global branch (gga_global_linear_fwd), per head, given its S and z:
 *   num_i = phi(q_i)^T S, den_i = phi(q_i) . z + eps, G_i = num_i / den_i,
 *   d num_i = dG_i / den_i, d den_i = -(dG_i . G_i) / den_i,
 *   d phi(q_i) = S d num_i + z d den_i,  dS = sum_i phi(q_i) d num_i^T,  dz = sum_i phi(q_i) d den_i,
 *   d phi(k_j) = dS v_j + dz,  d v_j = dS^T phi(k_j),  phi'(x) = 1 (x > 0) or e^x.
 * The results are ADDED to d_q, d_k, d_v (fp32 [n,H,r]), so the local branch's
 * gradients can be written there first.  Requires r <= 64.  dS, dz sums over nodes use
 * a fixed range order (deterministic).
 * g_fw (fp32 [n,H,r], device, may be NULL): the G this forward wrote.  num_i enters the
 * gradients only through dG_i . G_i; given g_fw, that term reads it and num_i is not
 * formed again (a third fewer matrix products); NULL forms it from S.  The two agree to
 * rounding.  Not checked against q, S, z: a G from other inputs gives other gradients.
 */
size_t gga_global_linear_bwd_workspace(int32_t n, int32_t heads, int32_t r);
int gga_global_linear_bwd(int32_t n, int32_t heads, int32_t r, const float *q, const float *k, const float *v,
                          float eps, const float *s, const float *z, const float *d_g, const float *g_fw,
                          float *d_q, float *d_k, float *d_v, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Batches of graphs ("Gated Local-Global Graph Attention", Implementation notes
 * note 1: a batched node input with one sparse adjacency list per graph).  The
 * graphs are packed along the node axis: graph b owns node rows node_ptr[b] ..
 * node_ptr[b+1]-1 (node_ptr int32 [batch+1], device, node_ptr[0] = 0,
 * non-decreasing, node_ptr[batch] = n; graphs may be empty).  The local branch
 * needs nothing new: on the block-diagonal edge list below, every softmax already
 * stays inside its graph.  The global branch's statistics become per graph.
 * node_ptr and edge_ptr are not checked on the host (they are device arrays); a
 * malformed one gives unspecified values but no access outside the buffers.
 * ------------------------------------------------------------------------ */

/*
 * Pack per-graph COO lists into one block-diagonal COO list over the packed node
 * axis: entries edge_ptr[b] .. edge_ptr[b+1]-1 (edge_ptr int32 [batch+1], device,
 * edge_ptr[batch] = e) belong to graph b and hold local ids in [0, n_b); they
 * become id + node_ptr[b].  An id outside [0, n_b) (or an entry outside every
 * graph's range) is written as -1 and counted in *d_bad (cleared first).  COO
 * order is kept.  src_local, dst_local, src, dst int32 [e].
 */
int gga_batch_edges(int32_t batch, const int32_t *node_ptr, const int32_t *edge_ptr, int64_t e,
                    const int32_t *src_local, const int32_t *dst_local, int32_t *src, int32_t *dst, int32_t *d_bad,
                    void *stream);

/*
 * Global branch per graph of a batch (gga_global_linear_fwd with the sums over j
 * taken over the rows of i's graph):
 *   S[b,h] = sum_{j in b} phi(k_j) v_j^T   fp32 [batch,H,r,r]
 *   z[b,h] = sum_{j in b} phi(k_j)         fp32 [batch,H,r]
 *   g[i,h,:] = phi(q_i)^T S[b,h] / (phi(q_i) . z[b,h] + eps)   for i in graph b.
 * An empty graph has S = 0, z = 0.  Deterministic.  s_out and z_out may be NULL.
 */
size_t gga_global_linear_batch_workspace(int32_t n, int32_t batch, int32_t heads, int32_t r);
int gga_global_linear_batch_fwd(int32_t n, int32_t batch, const int32_t *node_ptr, int32_t heads, int32_t r,
                                const float *q, const float *k, const float *v, float eps, float *s_out, float *z_out,
                                float *g_out, void *ws, size_t ws_bytes, void *stream);

/*
 * Its backward (gga_global_linear_bwd per graph, with s [batch,H,r,r] and
 * z [batch,H,r] from the forward, and g_fw as there): adds the gradients into d_q,
 * d_k, d_v.  Requires r <= 64.  Workspace: gga_global_linear_batch_workspace.
 */
int gga_global_linear_batch_bwd(int32_t n, int32_t batch, const int32_t *node_ptr, int32_t heads, int32_t r,
                                const float *q, const float *k, const float *v, float eps, const float *s,
                                const float *z, const float *d_g, const float *g_fw, float *d_q, float *d_k,
                                float *d_v, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * GAT variants the Tinymesh page ("Evidence and limits") lists as not yet
 * covered, read as in the GATConv its "Reference contract" section follows:
 * learned edge features in the score and head averaging.
 * ------------------------------------------------------------------------ */

/*
 * Additive local attention with an edge term: for edge e: u -> v and head h the
 * logit is z_e = s_src[u,h] + s_dst[v,h] + s_edge[e,h] before LeakyReLU (s_edge
 * fp32 [e,H] in COO order, e.g. a_e . (F W_e) per head from gga_gat_coef_fwd on the
 * edge features); otherwise as gga_local_attn_fwd in additive mode.  `eid` is the
 * COO index of each CSR position (gga_coo_to_csr).  fp32 hf only (GGA_EUNSUPPORTED
 * otherwise).  Deterministic.
 */
size_t gga_local_attn_fwd_edge_workspace(const gga_local_desc *d);
int gga_local_attn_fwd_edge(const gga_local_desc *d, const float *s_dst, const float *s_src, const void *hf,
                            const float *s_edge, const int32_t *row_ptr, const int32_t *col, const int32_t *eid,
                            const void *plan, float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * Its backward (as gga_local_attn_bwd in additive mode, with the same logits), plus
 * d_s_edge[e,h] = dz_e = ds_e LeakyReLU'(z_e), fp32 [e,H] in COO order.  eid and
 * eid_s are the COO indices of the CSR by destination and by source.
 */
size_t gga_local_attn_bwd_edge_workspace(const gga_local_desc *d);
int gga_local_attn_bwd_edge(const gga_local_desc *d, const float *s_dst, const float *s_src, const void *hf,
                            const float *s_edge, const float *out, const float *lse, const float *d_out,
                            const int32_t *row_ptr, const int32_t *col, const int32_t *eid, const void *plan,
                            const int32_t *row_ptr_s, const int32_t *col_s, const int32_t *eid_s, const void *plan_s,
                            float *d_s_dst, float *d_s_src, float *d_hf, float *d_s_edge, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Head averaging: out[n,c] = (1/H) sum_h in[n,h,c] (in fp32 [n,H,C], out [n,C]), and
 * its backward d_in[n,h,c] = d_out[n,c] / H.
 */
int gga_head_mean(int32_t n, int32_t heads, int32_t head_dim, const float *in, float *out, void *stream);
int gga_head_mean_bwd(int32_t n, int32_t heads, int32_t head_dim, const float *d_out, float *d_in, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GGA_H */
