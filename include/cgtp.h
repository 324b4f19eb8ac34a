/*
 * cgtp.h -- C ABI of libcgtp: the O(3)-equivariant Clebsch-Gordan tensor
 * product (CGTP), batched and fused with graph convolution, on AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed (sources are the pages this library follows):
 *  - "An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep
 *    Networks" (sciencestack.ai page), Abstract and Figure 1: a block-sparse
 *    real CG tensor contracted with two dense vectors, followed by a
 *    structured weight; Figure 4: use case A (batched rows) and use case B
 *    (graph convolution, node features combined with edge features and
 *    summed into the receiving node); the Abstract also names the gradient.
 *  - Sobek (aiqbench.com page, Abstract): the convolution is evaluated with
 *    bounded receiver-side state and no edge-sized intermediates, forward and
 *    backward.
 *  - LunaTP (readsearch.ai page, Abstract): node-centric execution.
 *  - OpenEquivariance discussion "The GPU memory optimization with Larger
 *    angular momentum": near-zero device memory overhead, only returned
 *    buffers are new, a deterministic convolution exists next to an atomic one.
 *
 * Conventions (readings; the pages fix none of them):
 *  - irreps strings "MULxLP" joined by '+', 0 <= L <= 7, P in {e,o}; blocks
 *    concatenated in string order; element (channel u, component m) of a
 *    block at offset + u*(2L+1) + (m+L);
 *  - real basis with l = 1 ordered (y, z, x); every CG block has Frobenius
 *    norm 1 and its first nonzero (row-major i, j, k) positive;
 *  - paths: i1 over input irreps, i2 over SH irreps, l3 ascending, parity
 *    p1*p2, kept if (l3, p3) occurs in the output; an output irrep that
 *    occurs once receives the sum of all paths producing it, one that occurs
 *    k > 1 times needs exactly k producing paths, taken in order;
 *  - uvu weights: per row/edge, the concatenation over paths of [mul];
 *    uvw weights (shared): the concatenation over paths of [mul_in][mul_out].
 *
 * Memory and streams: every device buffer is owned by the caller, must be a
 * device pointer to contiguous row-major data of the plan's dtype, aligned
 * to its element size, and outputs must not alias inputs.  The library
 * never allocates, frees or synchronises device memory; the entry points that
 * need temporary memory (cgtp_tp_backward and cgtp_conv_backward_ws for uvw,
 * cgtp_conv_backward_radial for dTheta) take it from the caller.  `stream` is a hipStream_t (NULL = the default
 * stream); all work is enqueued on it asynchronously.
 * Index arrays are int32 and N, E < 2^31.
 *
 * Errors: every entry point returns a cgtp_status; the message of the last
 * failure on the calling thread is cgtp_last_error().  Argument checks run
 * before any GPU call.  A kernel fault surfaces at the caller's next
 * synchronisation with the stream, not here.  No exception or abort crosses
 * the ABI.
 */
#ifndef CGTP_H
#define CGTP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cgtp_status {
    CGTP_OK = 0,
    CGTP_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, aliasing */
    CGTP_ERR_IRREPS = 2,      /* irreps string or path/slot rule violated      */
    CGTP_ERR_UNSUPPORTED = 3, /* valid request this build does not implement   */
    CGTP_ERR_COMPILE = 4,     /* hipRTC failed; the log is in cgtp_last_error  */
    CGTP_ERR_HIP = 5,         /* a HIP runtime call failed                     */
    CGTP_ERR_INTERNAL = 6
} cgtp_status;

typedef enum cgtp_mode { CGTP_UVU = 0, CGTP_UVW = 1 } cgtp_mode;
typedef enum cgtp_dtype { CGTP_F32 = 0, CGTP_F64 = 1 } cgtp_dtype;

typedef struct cgtp_plan cgtp_plan; /* opaque, immutable after creation */

typedef struct cgtp_plan_info {
    int32_t d_x;          /* width of one input row (node features)          */
    int32_t d_sh;         /* width of one edge/row of y (spherical harmonics) */
    int32_t d_out;        /* width of one output row                          */
    int32_t num_paths;
    int64_t weight_numel; /* uvu: weights per row/edge; uvw: shared total     */
    int32_t nnz_total;    /* CG nonzeros summed over paths                    */
    int32_t mode;         /* cgtp_mode                                        */
    int32_t dtype;        /* cgtp_dtype                                       */
    int32_t fwd_tasks;    /* waves per receiver in the forward convolution    */
} cgtp_plan_info;

typedef struct cgtp_path_info {
    int32_t i1, i2, slot;         /* input irrep, SH irrep, output block       */
    int32_t l1, l2, l3, p3;       /* degrees and output parity (+1/-1)         */
    int32_t x_off, y_off, out_off;/* block offsets in x, y and out rows        */
    int32_t mul_in, mul_out;
    int64_t w_off;                /* offset of this path's weights             */
    int32_t nnz;                  /* CG nonzeros of this path's block          */
} cgtp_path_info;

/*
 * Plan: parse the three irreps strings, enumerate the paths, compute the real
 * CG blocks (the planner's own exact code), drop the zeros (|C| <= 1e-9) and
 * generate one gfx950 module with the nonzeros as compile-time constants
 * (sciencestack.ai page, TL;DR and Abstract: JIT generation with static
 * analysis; OpenEquivariance discussion: nonzeros in the instruction stream).
 * The module is compiled with the ROCm installation's hipRTC
 * ($ROCM_PATH/lib/libhiprtc.so.7, or $CGTP_HIPRTC), loaded into a link
 * namespace of its own so that a hipRTC already in the process (one bundled
 * with a framework) does not take its place, or taken from the on-disk cache
 * ($CGTP_CACHE_DIR, default: a jit_cache folder next to the library; the key
 * names the compiler).  The module is loaded on a device at its first launch
 * there.  Allocates no device memory.
 * uvu needs mul_out == mul_in on every path; both modes need SH mul == 1.
 * Errors: CGTP_ERR_INVALID_ARG (null), CGTP_ERR_IRREPS, CGTP_ERR_COMPILE.
 */
cgtp_status cgtp_plan_create(const char *in_irreps, const char *sh_irreps, const char *out_irreps,
                             cgtp_mode mode, cgtp_dtype dtype, cgtp_plan **plan_out);
/*
 * Release a plan and the code objects it loaded on any device.  Not on the
 * pages: every object that cgtp_plan_create hands out needs an owner-side
 * release, and the only device resources a plan holds are its loaded modules
 * (the OpenEquivariance discussion's rule that the library keeps no device
 * buffers of its own).  The caller must not use the plan afterwards, and must
 * first let every kernel launched with it finish (synchronise the streams it
 * used): the code those kernels run is unloaded here.  NULL is accepted and
 * ignored.  Unloading errors are not reported; always returns CGTP_OK.
 */
cgtp_status cgtp_plan_destroy(cgtp_plan *plan);
/*
 * Plan bookkeeping for sizing caller-owned buffers: widths d_x, d_sh, d_out,
 * path count, weight count, CG nonzeros (sciencestack.ai page, Figure 1: the
 * dense operands x, y, the output and the structured weight W whose sizes
 * follow from the irreps; Figure 2: the sparse blocks).  The name carries
 * `_get` because the C struct cgtp_plan_info already owns the plain name.
 * Host only.  Errors: CGTP_ERR_INVALID_ARG (NULL).
 */
cgtp_status cgtp_plan_info_get(const cgtp_plan *plan, cgtp_plan_info *info);
/* One path of the plan (input irrep, SH irrep, output block, degrees, offsets, nonzeros;
 * sciencestack.ai page, Figure 1: one sparse block per coupling path).  Host only.
 * Errors: CGTP_ERR_INVALID_ARG (NULL, path out of range). */
cgtp_status cgtp_plan_path(const cgtp_plan *plan, int32_t path, cgtp_path_info *info);
/* Copies up to `cap` nonzeros of one path's real CG block: ijk[3*n] (i, j, k)
 * and values[n] as float64.  *nnz receives the full count. */
cgtp_status cgtp_plan_path_coefficients(const cgtp_plan *plan, int32_t path, int32_t cap,
                                        int32_t *ijk, double *values, int32_t *nnz);
/* The generated HIP source of the plan's module (owned by the plan). */
const char *cgtp_plan_source(const cgtp_plan *plan);
/*
 * Waves per receiver row that a receiver-owned pass launches for a graph of N
 * receivers and E edges (LunaTP page, Abstract: node-centric execution; the
 * split spreads one node's edges over several waves): pass 0 = the forward
 * (cgtp_conv_forward, cgtp_conv_forward_ordered), pass 1 = the receiver pass
 * of cgtp_conv_double_backward.  *split receives 1, 2 or 4; the kernel that
 * runs is cgtp_conv_fwd / cgtp_conv_dbwd_recv with the suffix _split2 or
 * _split4 when *split > 1.  The parts of a row are summed in part order, so
 * the bits depend only on the plan, N and E.  Uses no device.
 * Errors: CGTP_ERR_INVALID_ARG (NULL, pass not 0 or 1, N or E out of range).
 */
cgtp_status cgtp_conv_row_split(const cgtp_plan *plan, int64_t N, int64_t E, int32_t pass, int32_t *split);

/*
 * Batched tensor product, use case A (sciencestack.ai page, Figure 4A):
 *   uvu: out[b, o + u(2l3+1) + k] = sum_paths W[b, w_p + u] *
 *                                   sum_{i,j} C[i,j,k] x[b, a + u(2l1+1) + i] y[b, b_p + j]
 *        w is [B][weight_numel], shared_weights must be 0;
 *   uvw: out[b, o + v(2l3+1) + k] = sum_paths sum_u W_p[u][v] * (same contraction)
 *        w is the shared [weight_numel] block, shared_weights must be 1; output
 *        multiplicities above 16 run as 16-wide tiles of output channels.
 * x [B][d_x], y [B][d_sh], out [B][d_out] (overwritten).  B = 0 is a no-op.
 */
cgtp_status cgtp_tp_forward(const cgtp_plan *plan, int64_t B, const void *x, const void *y,
                            const void *w, int shared_weights, void *out, void *stream);

/*
 * Batched tensor product backward, use case A (sciencestack.ai page, Abstract:
 * gradient kernels; Figure 4A): with g = grad_out [B][d_out],
 *   uvu (shared_weights = 0), per row b:
 *     grad_w[b, w_p + u] = sum_{ijk} C x[b,u,i] y[b,j] g[b,u,k]
 *     grad_y[b, b_p + j] = sum_p sum_u W[b,p,u] sum_{ik} C x[b,u,i] g[b,u,k]
 *     grad_x[b, a_p + u(2l1+1) + i] = sum_p W[b,p,u] sum_{jk} C y[b,j] g[b,u,k]
 *   uvw (shared_weights = 1), with G_p[b,u,k] = sum_w W_p[u][w] g[b, o_p + w(2l3+1) + k]:
 *     grad_x[b, a_p + u(2l1+1) + i] = sum_p sum_{jk} C y[b,j] G_p[b,u,k]
 *     grad_y[b, b_p + j] = sum_p sum_u sum_{ik} C x[b,u,i] G_p[b,u,k]
 *     grad_w[w_p + u*mul_out + w] = sum_b sum_{ijk} C x[b,u,i] y[b,j] g[b, o_p + w(2l3+1) + k]
 *   The shared-weight gradient sums over all rows: per-chunk partials go to
 *   the caller's `workspace` (workspace_bytes >= cgtp_tp_backward_workspace_size;
 *   0 for uvu, where workspace may be NULL) and are summed in chunk order.
 *   A uvw plan with a multiplicity above 16 runs the uvw convolution backward
 *   (cgtp_conv_backward_ws) on the identity graph, row b being the edge from
 *   sender b to receiver b; its workspace (256-byte aligned) then holds that
 *   call's workspace and the index array 0..B, and is needed for every gradient.
 * Any of grad_x / grad_y / grad_w may be NULL to skip it; outputs are
 * overwritten, one owner per element, no atomics, bitwise deterministic.
 * B = 0 writes nothing, except that a uvw grad_w is set to zero.
 */
cgtp_status cgtp_tp_backward_workspace_size(const cgtp_plan *plan, int64_t B, size_t *bytes);
/* uvw: the backward kernels form their own module, generated and compiled on the first call;
 * this builds it ahead of time (host only) and cgtp_plan_uvw_backward_source returns its source
 * (owned by the plan; NULL before it exists). */
cgtp_status cgtp_plan_uvw_backward_prepare(const cgtp_plan *plan);
const char *cgtp_plan_uvw_backward_source(const cgtp_plan *plan);
cgtp_status cgtp_tp_backward(const cgtp_plan *plan, int64_t B, const void *x, const void *y, const void *w,
                             int shared_weights, const void *grad_out, void *grad_x, void *grad_y, void *grad_w,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * The batched backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and bits as
 * cgtp_tp_backward; the temporary memory it needs (the uvw shared-weight
 * gradient's per-chunk partials, or the identity-graph route of plans with a
 * multiplicity above 16) comes from a fixed 64 MiB device array inside the
 * library, one per device, held until the process ends.  Calls whose
 * workspace need (cgtp_tp_backward_workspace_size) exceeds 64 MiB return
 * CGTP_ERR_UNSUPPORTED.  The first call on a device looks up that device's
 * copy of the array (and, as for every entry point, loads the plan's code on
 * the device); later calls allocate nothing.  Every call on one device shares
 * the same array: calls that overlap in time on one device (different streams
 * or threads) race and give unspecified results; calls ordered on one stream
 * are safe.  uvu plans use no scratch.
 */
cgtp_status cgtp_tp_backward_noalloc(const cgtp_plan *plan, int64_t B, const void *x, const void *y, const void *w,
                                     int shared_weights, const void *grad_out, void *grad_x, void *grad_y,
                                     void *grad_w, void *stream);

/*
 * Fused convolution forward, use case B (sciencestack.ai page, Figure 4B;
 * Sobek page, Abstract): for every receiver n,
 *   out[n] = sum_{e in [row_ptr[n], row_ptr[n+1])} TP_uvu(x[col[e]], y[e], W[e]).
 * row_ptr [N+1] and col [E] form a receiver-sorted CSR (row_ptr[0] = 0,
 * non-decreasing, row_ptr[N] = E, 0 <= col < N); y [E][d_sh] and w
 * [E][weight_numel] are in CSR edge order; x [N][d_x]; out [N][d_out] is
 * overwritten, receivers without edges get zeros.  One owner per output row:
 * no atomics, bitwise deterministic (when a row is split over several waves,
 * cgtp_conv_row_split, its parts are added in a fixed order).  uvw plans (fully connected multiplicity
 * mixing inside the convolution; Sobek page, Abstract): w is the shared
 * [weight_numel] block instead, out[n] = sum_e TP_uvw(x[col[e]], y[e], W),
 * the mixing running on MFMA per tile of 16 receivers.
 */
cgtp_status cgtp_conv_forward(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                              const int32_t *col, const void *x, const void *y, const void *w,
                              void *out, void *stream);

/*
 * Same as cgtp_conv_forward with a receiver schedule: order [N] is a
 * permutation of the receivers giving the order in which their rows are
 * started (NULL = natural order).  The result does not depend on it (each
 * receiver is still summed by one owner in CSR edge order); a heavy-first
 * order shortens the tail on power-law graphs (LunaTP page, Abstract:
 * node-centric execution).  The caller must pass a permutation of 0..N-1.
 */
cgtp_status cgtp_conv_forward_ordered(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                      const int32_t *col, const int32_t *order, const void *x, const void *y,
                                      const void *w, void *out, void *stream);

/*
 * Fused convolution with radially projected weights (Sobek page, Abstract:
 * the radial projection reassociated with the coupling and the aggregation,
 * so that edge-sized weights are never stored): for a uvu plan,
 *   W_e = rho[e] @ Theta,   out[n] = sum_e TP_uvu(x[col[e]], y[e], W_e),
 * with rho [E][R] the edges' radial features (CSR edge order) and Theta
 * [R][weight_numel] shared.  Each edge reads R values instead of weight_numel;
 * each workgroup copies to LDS the Theta columns of one path group's channel
 * tile (R x paths x tile width elements must fit the 160 KB of a workgroup,
 * else CGTP_ERR_UNSUPPORTED before any GPU work).  1 <= R <= 64.  The kernel for a given R is generated
 * and compiled on the first call with that R (then cached).  Everything else
 * (CSR, schedule `order`, layouts, determinism) as cgtp_conv_forward_ordered.
 *
 * For a uvw plan (the fully connected family of the same passage) each edge
 * has its own blocks W_e,p[u][w] = sum_r rho[e][r] Theta[r][w_p + u mul_out + w],
 * out[n] = sum_e TP_uvw(x[col[e]], y[e], W_e).  The coupling is linear in y, so
 * radial channel r contributes the shared-weight uvw convolution of
 * rho[:, r] * y with Theta's row r: R launch rounds of the uvw convolution
 * kernel (the scaling done as each edge's SH values are loaded; channel 0
 * writes `out`, the others add, in order), with no per-edge weights formed
 * and no workspace.  CGTP_ERR_UNSUPPORTED when the plan's uvw convolution is
 * unsupported (cgtp_conv_forward_ordered's LDS limit).  cgtp_plan_radial_prepare then
 * compiles the uvw convolution module (any R) and cgtp_plan_radial_source
 * returns its source.
 */
/* Generate and compile the radial kernel for R now (host only, no device needed), e.g. to
 * move the JIT cost out of the first call; its source is then cgtp_plan_radial_source (owned
 * by the plan; NULL before the module for R exists). */
cgtp_status cgtp_plan_radial_prepare(const cgtp_plan *plan, int32_t R);
const char *cgtp_plan_radial_source(const cgtp_plan *plan, int32_t R);
cgtp_status cgtp_conv_forward_radial(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                     const int32_t *col, const int32_t *order, const void *x, const void *y, int32_t R,
                                     const void *rho, const void *theta, void *out, void *stream);

/*
 * Backward of the radially projected convolution (Sobek page, Abstract: the
 * reassociation extends through the backward; no edge-sized weights or
 * adjoints).  With W_e = rho[e] @ Theta and (dx, dy, dW_e) the gradients of
 * cgtp_conv_backward for that W:
 *   grad_x [N][d_x], grad_y [E][d_sh]   as cgtp_conv_backward,
 *   grad_rho [E][R]                     = dW_e Theta^T  (per edge),
 *   grad_theta [R][weight_numel]        = sum_e rho[e]^T dW_e.
 * One sender-ordered pass over the transpose (cgtp_graph_transpose) per path
 * group: W_e is rebuilt from rho and the LDS copy of Theta, and dW_e is
 * consumed at once into grad_rho (summed over the channel lanes) and into
 * registers holding the dTheta sums of a chunk of consecutive senders.  Each
 * chunk writes one partial to `workspace` (at least
 * cgtp_conv_backward_radial_workspace_size bytes, 256-byte aligned,
 * caller-owned, contents ignored on entry), summed in chunk order; neither W_e
 * nor dW_e is stored.  Any output may be NULL to skip it (the workspace is
 * needed only for grad_theta); outputs are overwritten, no atomics, bitwise
 * deterministic.  N = 0 sets grad_theta to zero.  1 <= R <= 64;
 * CGTP_ERR_UNSUPPORTED when one path group's Theta columns (R x its channels)
 * and the reduction buffer do not fit one workgroup's 160 KB of LDS.
 *
 * uvw plans, radial channel by channel (ys = rho[:, r] * y, G_r = Theta_r^T g
 * per receiver): dTheta_r is the uvw weight-gradient pass on (x, ys) (tile
 * partials summed in tile order), the unit-weight sender pass on (x, ys, G_r)
 * adds channel r's share to grad_x and yields t = d/dys, folded into
 * grad_y += rho[:, r] t and grad_rho[:, r] = <y, t> (channel 0 writes).  The
 * workspace is needed whenever N > 0 (any output requested): G, R x
 * ceil(N / 16) dTheta partials and two E x d_sh rows (the scaled SH and t),
 * each part 256-byte aligned; cgtp_conv_backward_radial_workspace_size gives
 * the total.  No per-edge weight or weight gradient is formed.
 */
cgtp_status cgtp_conv_backward_radial_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, int32_t R,
                                                    size_t *bytes);
cgtp_status cgtp_conv_backward_radial(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                      const int32_t *col, const int32_t *t_row_ptr, const int32_t *t_edge,
                                      const int32_t *t_dst, const void *x, const void *y, int32_t R, const void *rho,
                                      const void *theta, const void *grad_out, void *grad_x, void *grad_y,
                                      void *grad_rho, void *grad_theta, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * Heavy-first receiver schedule, once per graph (LunaTP page, Abstract:
 * node-centric execution; here it orders which receivers the node-owned
 * waves start first, so that the heaviest nodes of a power-law graph do not
 * finish last).  order [N] (caller-owned) receives the receivers stably sorted
 * by floor(log2(in-degree + 1)), largest first (ties keep node order).
 * row_ptr as in cgtp_conv_forward.  Integer result, deterministic, enqueued on
 * `stream`.  N = 0 is a no-op.  Errors: CGTP_ERR_INVALID_ARG (NULL,
 * misaligned, N out of range), CGTP_ERR_HIP (launch).
 */
cgtp_status cgtp_graph_order(int64_t N, const int32_t *row_ptr, int32_t *order, void *stream);

/*
 * Sender-sorted transpose of a receiver CSR, once per graph.  It is what
 * makes the backward deterministic without atomics or input-sized scratch:
 * the OpenEquivariance discussion contrasts an atomic fused convolution with a
 * deterministic one that needs scratch space; here the gradient of each sender
 * row has one owner that walks its edges through this index (Sobek page,
 * Abstract: adjoints without edge-sized intermediates).  Outputs:
 * t_row_ptr [N+1], t_edge [E] (edge ids grouped by sender, ascending edge id
 * inside a sender: a stable sort by col) and t_dst [E] (receiver of
 * t_edge[t]).  Integer results, bit-exact and deterministic, enqueued on
 * `stream`.  All outputs caller-owned, disjoint from the inputs.  Errors:
 * CGTP_ERR_INVALID_ARG (NULL, misaligned, N or E out of range), CGTP_ERR_HIP.
 */
cgtp_status cgtp_graph_transpose(int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col,
                                 int32_t *t_row_ptr, int32_t *t_edge, int32_t *t_dst, void *stream);

/*
 * Fused convolution backward (sciencestack.ai page, Abstract: gradient
 * kernels; Sobek page: adjoints without edge-sized intermediates).  With
 * g = grad_out [N][d_out], for each edge e = (s -> n) and path p:
 *   grad_w[e, w_p + u] = sum_{ijk} C x[s,u,i] y[e,j] g[n,u,k]
 *   grad_y[e, b_p + j] = sum_p sum_u W[e,p,u] sum_{ik} C x[s,u,i] g[n,u,k]
 *   grad_x[s, a_p + u(2l1+1) + i] = sum_{e: col[e]=s} sum_p W[e,p,u] sum_{jk} C y[e,j] g[n,u,k]
 * One pass in sender order over the transpose (cgtp_graph_transpose): each
 * output row has one owner, no atomics, bitwise deterministic.  Any of
 * grad_x / grad_y / grad_w may be NULL to skip it; outputs are overwritten.
 */
cgtp_status cgtp_conv_backward(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                               const int32_t *col, const int32_t *t_row_ptr, const int32_t *t_edge,
                               const int32_t *t_dst, const void *x, const void *y, const void *w,
                               const void *grad_out, void *grad_x, void *grad_y, void *grad_w,
                               void *stream);

/*
 * Fused convolution backward in receiver order (uvu plans): the same results
 * as cgtp_conv_backward, from a schedule whose per-edge gather is the sender
 * row x[col[e]] (d_x wide) instead of the receiver's output-gradient row
 * (d_out wide).  Sources: sciencestack.ai page, Abstract (gradient kernels
 * that minimise global reads and writes); LunaTP page, Abstract
 * (node-centric execution: the output gradient of a node stays in
 * registers while its edges stream past); OpenEquivariance discussion
 * (a deterministic convolution uses a bounded scratch buffer instead of
 * atomics).  The edges are taken in contiguous ranges [e_lo, e_hi) of the
 * receiver CSR; for each range:
 *   1. one pass over its edges (one wave per block of consecutive edges, the
 *      receiver's gradient row held in registers) writes grad_w and grad_y
 *      of every edge (formulas of cgtp_conv_backward) and, when grad_x is
 *      wanted, the edge's contribution to its sender's dx,
 *        h[e - e_lo, a_p + u(2l1+1) + i] = sum_p W[e,p,u] sum_{jk} C y[e,j] g[n,u,k],
 *      into `workspace` ([e_hi - e_lo][d_x] rows);
 *   2. for every sender, the rows of its edges in the range are summed in
 *      ascending edge id (from the transpose) into grad_x: the first range
 *      writes, later ranges add.
 * The range length is the number of rows the workspace holds (at most E):
 * the workspace is a caller-chosen, bounded buffer, independent of E when
 * the caller wants it to be; a smaller one means more ranges and more
 * read-modify-write of grad_x.  cgtp_conv_backward_receiver_workspace_size
 * gives *bytes = E * d_x * elem (one range) and *min_bytes, the least the call
 * accepts (one block of edges).  workspace: 256-byte aligned, caller-owned,
 * disjoint from every argument, contents ignored on entry, unspecified on
 * return; needed only when grad_x is wanted and E > 0.  t_row_ptr and t_edge
 * are those of cgtp_graph_transpose (t_dst is not needed); they may be NULL
 * when grad_x is NULL.  Any gradient may be NULL to skip it; outputs are
 * overwritten, each element has one owner, no atomics, bitwise deterministic
 * for a given workspace size (the range boundaries group the dx sums).
 * Errors: CGTP_ERR_INVALID_ARG (NULL, misaligned, overlapping, workspace
 * below *min_bytes), CGTP_ERR_UNSUPPORTED (uvw plans), CGTP_ERR_HIP.
 */
cgtp_status cgtp_conv_backward_receiver_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, size_t *bytes,
                                                       size_t *min_bytes);
cgtp_status cgtp_conv_backward_receiver(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                        const int32_t *col, const int32_t *t_row_ptr, const int32_t *t_edge,
                                        const void *x, const void *y, const void *w, const void *grad_out,
                                        void *grad_x, void *grad_y, void *grad_w, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * Fused convolution backward with a caller workspace; needed by uvw plans
 * (shared [weight_numel] W, fully connected multiplicity mixing inside the
 * convolution; Sobek page, Abstract: gradients of the same operator without
 * edge-sized intermediates).  With g = grad_out [N][d_out] and, per receiver
 * n and path p, G_p[n,u,k] = sum_w W_p[u][w] g[n, o_p + w(2l3+1) + k]:
 *   grad_x[s, a_p + u(2l1+1) + i] = sum_{e: col[e]=s} sum_p sum_{jk} C y[e,j] G_p[n_e,u,k]
 *   grad_y[e, b_p + j]            = sum_p sum_u sum_{ik} C x[col[e],u,i] G_p[n_e,u,k]
 *   grad_w[w_p + u*mul_out + w]   = sum_n sum_k T_p[n,u,k] g[n, o_p + w(2l3+1) + k],
 *     T_p[n,u,k] = sum_{e into n} sum_{ij} C x[col[e],u,i] y[e,j]
 * (n_e the receiver of edge e).  G is computed per 16-receiver tile on MFMA
 * into the workspace, then read by one sender-ordered pass over the transpose
 * (grad_x, grad_y: one owner per row); grad_w is one partial per 16-receiver
 * tile (the forward's edge pass, then MFMA over the tile's receivers) summed
 * in tile order.  No atomics, bitwise deterministic.  `order` is the receiver
 * schedule of the grad_w pass (as in cgtp_conv_forward_ordered, NULL =
 * natural); it decides which receivers share a tile, so grad_w's rounding (not
 * its value) depends on it, while grad_x and grad_y do not.  workspace: device memory of at
 * least cgtp_conv_backward_workspace_size(plan, N, E) bytes, 256-byte
 * aligned, caller-owned, disjoint from every argument; its contents on entry
 * are ignored and on return unspecified.  Any of grad_x / grad_y / grad_w may
 * be NULL to skip it; outputs are overwritten; N = 0 sets grad_w to zero.
 * uvu plans: identical to cgtp_conv_backward (order and workspace unused,
 * size 0).  The uvw backward kernels are generated and compiled on the first
 * call (then cached); cgtp_plan_conv_uvw_backward_prepare does it ahead of
 * time on the host, and cgtp_plan_conv_uvw_backward_source returns the
 * sources (module 0: G and grad_w kernels; 1: the sender pass; owned by the
 * plan, NULL before they exist).
 */
cgtp_status cgtp_conv_backward_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, size_t *bytes);
cgtp_status cgtp_conv_backward_ws(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                  const int32_t *col, const int32_t *order, const int32_t *t_row_ptr,
                                  const int32_t *t_edge, const int32_t *t_dst, const void *x, const void *y,
                                  const void *w, const void *grad_out, void *grad_x, void *grad_y, void *grad_w,
                                  void *workspace, size_t workspace_bytes, void *stream);
cgtp_status cgtp_plan_conv_uvw_backward_prepare(const cgtp_plan *plan);
const char *cgtp_plan_conv_uvw_backward_source(const cgtp_plan *plan, int32_t module);

/*
 * Fused convolution double backward: the higher partial derivatives used for
 * interatomic forces (sciencestack.ai page, Abstract; OpenEquivariance
 * discussion: a convolution double backward with four results; Sobek page,
 * Abstract: the same operator through double backward; LunaTP page,
 * Abstract: higher-order derivatives).  With (dx, dy, dW) the results of
 * cgtp_conv_backward for (x, y, w, grad_out) and upstream gradients gg_x
 * [N][d_x], gg_y [E][d_sh], gg_w [E][weight_numel] for them, the scalar
 *   L2 = <gg_x, dx> + <gg_y, dy> + <gg_w, dW>
 * is differentiated:
 *   grad_grad_out [N][d_out] = conv(gg_x, y, w) + conv(x, gg_y, w) + conv(x, y, gg_w)
 *   grad_x [N][d_x]          = sum over e = (s -> n): sum_p sum_{jk} C g[n,u,k] (W gg_y_j + gg_w y_j)
 *   grad_y [E][d_sh]         = sum_p sum_u sum_{ik} C g[n,u,k] (W gg_x[s,u,i] + gg_w x[s,u,i])
 *   grad_w [E][weight_numel] = sum_{ijk} C g[n,u,k] (gg_x[s,u,i] y_j + x[s,u,i] gg_y_j)
 * (conv(.) is cgtp_conv_forward; sums per path p and channel u as in
 * cgtp_conv_backward.)  grad_grad_out comes from one receiver-ordered pass
 * (schedule `order` as in cgtp_conv_forward_ordered, NULL = natural); the
 * other three from one sender-ordered pass over the transpose.  Any output may
 * be NULL to skip it (a pass with no requested output is not launched);
 * outputs are overwritten, each row has one owner, no atomics, bitwise
 * deterministic.  Every input named in a requested pass must be non-NULL
 * (pass zeros for an absent upstream gradient); x and gg_x always.  uvu plans;
 * uvw plans take cgtp_conv_double_backward_ws (CGTP_ERR_UNSUPPORTED here).
 */
cgtp_status cgtp_conv_double_backward(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                      const int32_t *col, const int32_t *order, const int32_t *t_row_ptr,
                                      const int32_t *t_edge, const int32_t *t_dst, const void *x, const void *y,
                                      const void *w, const void *grad_out, const void *gg_x, const void *gg_y,
                                      const void *gg_w, void *grad_x, void *grad_y, void *grad_w,
                                      void *grad_grad_out, void *stream);

/*
 * Convolution double backward with a caller workspace, for both operator
 * families (Sobek page, Abstract: the fully connected multiplicity mixing is
 * carried through forward, backward and double backward; sciencestack.ai
 * page, Abstract: higher partial derivatives).  uvu plans: exactly
 * cgtp_conv_double_backward (workspace unused, size 0).  uvw plans (shared W,
 * gg_w shaped like W, grad_w [weight_numel]): with G_p = W_p^T g and
 * G'_p = gg_w_p^T g per receiver (as in cgtp_conv_backward_ws),
 *   grad_x         = dx(y -> gg_y, G) + dx(y, G')
 *   grad_y         = dY(x -> gg_x, G) + dY(x, G')
 *   grad_w         = dW(T of (gg_x, y)) + dW(T of (x, gg_y))
 *   grad_grad_out  = conv(gg_x, y, W) + conv(x, gg_y, W) + conv(x, y, gg_w)
 * where dx, dY, dW and T are those of cgtp_conv_backward_ws and conv is the
 * uvw forward: the derivatives of <gg_x, dx> + <gg_y, dY> + <gg_w, dW>.  Each
 * sum is formed in a fixed order (the second and third terms added by later
 * launches of the same kernels; grad_w through per-tile partials summed in
 * order): no atomics, bitwise deterministic.  workspace: at least
 * cgtp_conv_double_backward_workspace_size bytes (G and G' for N receivers,
 * then two dW partials per 16-receiver tile), 256-byte aligned, caller-owned,
 * disjoint from every argument; needed unless only grad_grad_out is asked.
 * Inputs: x, gg_x, w, gg_w and grad_out always, y and gg_y when E > 0; `order`
 * is the receiver schedule of the receiver-tile passes (NULL = natural).  Any
 * output may be NULL to skip it; N = 0 sets grad_w to zero.
 * Errors: as cgtp_conv_backward_ws.
 */
cgtp_status cgtp_conv_double_backward_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, size_t *bytes);
cgtp_status cgtp_conv_double_backward_ws(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                         const int32_t *col, const int32_t *order, const int32_t *t_row_ptr,
                                         const int32_t *t_edge, const int32_t *t_dst, const void *x, const void *y,
                                         const void *w, const void *grad_out, const void *gg_x, const void *gg_y,
                                         const void *gg_w, void *grad_x, void *grad_y, void *grad_w,
                                         void *grad_grad_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Real spherical harmonics of the edge vectors, component normalisation
 * (sum_m Y_lm^2 = 2l+1, Y_1 = sqrt3 (y, z, x)/|r|), degrees 0..lmax (<= 7):
 * vec [E][3] (any nonzero length), y [E][(lmax+1)^2] overwritten.  These
 * are the edge features of the convolution (sciencestack.ai page, Figure 4B).
 */
cgtp_status cgtp_spherical_harmonics(int32_t lmax, cgtp_dtype dtype, int64_t E, const void *vec,
                                     void *y, void *stream);

/*
 * Message of the last failed call on this thread ("" if none).  Not on the
 * pages: a C ABI cannot carry exceptions, so every entry point returns a
 * status and leaves its reason here (for CGTP_ERR_COMPILE, the hipRTC log).
 * The string is owned by the library and valid until the next failing call on
 * the same thread.
 */
const char *cgtp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CGTP_H */
