/*
 * Explicit-loop CPU oracle for the fused CG tensor-product convolution.
 *
 * TEST INFRASTRUCTURE ONLY: called by the test-suite, the smoke check and the
 * cpu_baseline leg of the benchmark through oracle/loops.py.  The product
 * library never links or calls it.
 *
 * What is computed: "An Efficient Sparse Kernel Generator for O(3)-Equivariant
 * Deep Networks" (sciencestack.ai page), Abstract and Figures 1 and 4: per edge
 * (or batch row) the block-sparse CG tensor is contracted with the sender's
 * features x and the edge features y, each path is scaled by that edge's
 * weights, and messages are summed into the receiving node.  The formulas are
 * the ones written out in oracle/ref.py; here they are plain nested loops:
 * rows -> edges -> paths -> channels -> CG nonzeros, accumulated in double.
 *
 * Inputs may be float32 or float64 (flag in_f32); they are read and widened to
 * double exactly.  Outputs are double.  The path table has PT_FIELDS ints per
 * path (offsets into x, y, out, block sizes, multiplicities, weight offset and
 * the slice of the nonzero arrays).  OpenMP splits the outer loop only; each
 * output element is still summed in edge order by one thread.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { PT_A, PT_B, PT_O, PT_N1, PT_N2, PT_N3, PT_MUL_IN, PT_MUL_OUT, PT_WOFF, PT_NZ0, PT_NZN, PT_FIELDS };

static inline double ld(const void *p, size_t i, int f32)
{
    return f32 ? (double)((const float *)p)[i] : ((const double *)p)[i];
}

/* out[r, :] = sum over edges e in [ptr[r], ptr[r+1]) of the uvu product of
 * x[col[e]], y[e] and w[e].  With ptr[r] = r and col[r] = r this is the
 * batched product (use case A). */
int oracle_uvu_forward(int n_paths, const int *pt, const int *nzi, const int *nzj, const int *nzk,
                       const double *nzc, int d_x, int d_sh, int d_out, int w_row, int64_t n_rows,
                       const int64_t *ptr, const int64_t *col, const void *x, const void *y,
                       const void *w, int in_f32, double *out, int n_threads)
{
#pragma omp parallel for schedule(dynamic, 4) num_threads(n_threads)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *o = out + (size_t)r * d_out;
        memset(o, 0, sizeof(double) * (size_t)d_out);
        for (int64_t e = ptr[r]; e < ptr[r + 1]; ++e) {
            int64_t s = col[e];
            for (int p = 0; p < n_paths; ++p) {
                const int *q = pt + p * PT_FIELDS;
                for (int u = 0; u < q[PT_MUL_IN]; ++u) {
                    double wv = ld(w, (size_t)e * w_row + q[PT_WOFF] + u, in_f32);
                    for (int z = q[PT_NZ0]; z < q[PT_NZ0] + q[PT_NZN]; ++z) {
                        double xv = ld(x, (size_t)s * d_x + q[PT_A] + u * q[PT_N1] + nzi[z], in_f32);
                        double yv = ld(y, (size_t)e * d_sh + q[PT_B] + nzj[z], in_f32);
                        o[q[PT_O] + u * q[PT_N3] + nzk[z]] += wv * nzc[z] * xv * yv;
                    }
                }
            }
        }
    }
    return 0;
}

/* Edge gradients of sum(g * out): for every edge e of row r (g row r),
 *   dw[e, woff + u] = sum c * x[s,u,i] * y[e,j] * g[r,u,k]
 *   dy[e, b + j]    = sum over paths, u of c * w[e,p,u] * x[s,u,i] * g[r,u,k] */
int oracle_uvu_backward_edges(int n_paths, const int *pt, const int *nzi, const int *nzj,
                              const int *nzk, const double *nzc, int d_x, int d_sh, int d_out,
                              int w_row, int64_t n_rows, const int64_t *ptr, const int64_t *col,
                              const void *x, const void *y, const void *w, const void *g,
                              int in_f32, double *dy, double *dw, int n_threads)
{
#pragma omp parallel for schedule(dynamic, 4) num_threads(n_threads)
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int64_t e = ptr[r]; e < ptr[r + 1]; ++e) {
            int64_t s = col[e];
            memset(dy + (size_t)e * d_sh, 0, sizeof(double) * (size_t)d_sh);
            memset(dw + (size_t)e * w_row, 0, sizeof(double) * (size_t)w_row);
            for (int p = 0; p < n_paths; ++p) {
                const int *q = pt + p * PT_FIELDS;
                for (int u = 0; u < q[PT_MUL_IN]; ++u) {
                    double wv = ld(w, (size_t)e * w_row + q[PT_WOFF] + u, in_f32);
                    for (int z = q[PT_NZ0]; z < q[PT_NZ0] + q[PT_NZN]; ++z) {
                        double xv = ld(x, (size_t)s * d_x + q[PT_A] + u * q[PT_N1] + nzi[z], in_f32);
                        double yv = ld(y, (size_t)e * d_sh + q[PT_B] + nzj[z], in_f32);
                        double gv = ld(g, (size_t)r * d_out + q[PT_O] + u * q[PT_N3] + nzk[z], in_f32);
                        dw[(size_t)e * w_row + q[PT_WOFF] + u] += nzc[z] * xv * yv * gv;
                        dy[(size_t)e * d_sh + q[PT_B] + nzj[z]] += nzc[z] * wv * xv * gv;
                    }
                }
            }
        }
    }
    return 0;
}

/* Sender gradient: for sender row r, dx[r, a + u*n1 + i] = sum over its edges t in
 * [sptr[r], sptr[r+1]) of c * w[t,p,u] * y[t,j] * g[gidx[t],u,k], where the edge rows of
 * y and w are given in the sender's order and gidx[t] picks the receiver's g row. */
int oracle_uvu_backward_x(int n_paths, const int *pt, const int *nzi, const int *nzj,
                          const int *nzk, const double *nzc, int d_x, int d_sh, int d_out,
                          int w_row, int64_t n_rows, const int64_t *sptr, const int64_t *gidx,
                          const void *y, const void *w, const void *g, int in_f32, double *dx,
                          int n_threads)
{
#pragma omp parallel for schedule(dynamic, 4) num_threads(n_threads)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *d = dx + (size_t)r * d_x;
        memset(d, 0, sizeof(double) * (size_t)d_x);
        for (int64_t t = sptr[r]; t < sptr[r + 1]; ++t) {
            int64_t n = gidx[t];
            for (int p = 0; p < n_paths; ++p) {
                const int *q = pt + p * PT_FIELDS;
                for (int u = 0; u < q[PT_MUL_IN]; ++u) {
                    double wv = ld(w, (size_t)t * w_row + q[PT_WOFF] + u, in_f32);
                    for (int z = q[PT_NZ0]; z < q[PT_NZ0] + q[PT_NZN]; ++z) {
                        double yv = ld(y, (size_t)t * d_sh + q[PT_B] + nzj[z], in_f32);
                        double gv = ld(g, (size_t)n * d_out + q[PT_O] + u * q[PT_N3] + nzk[z], in_f32);
                        d[q[PT_A] + u * q[PT_N1] + nzi[z]] += nzc[z] * wv * yv * gv;
                    }
                }
            }
        }
    }
    return 0;
}

/* Batched uvw product (use case A, shared weights): for each row r and path p,
 *   t[u,k] = sum c * x[r,u,i] * y[r,j];  out[r, o + w*n3 + k] += sum_u t[u,k] * W_p[u,w]. */
int oracle_uvw_forward(int n_paths, const int *pt, const int *nzi, const int *nzj, const int *nzk,
                       const double *nzc, int d_x, int d_sh, int d_out, int64_t n_rows,
                       const void *x, const void *y, const void *w, int in_f32, double *out,
                       int n_threads)
{
#pragma omp parallel for schedule(dynamic, 4) num_threads(n_threads)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *o = out + (size_t)r * d_out;
        double t[16 * 64];
        memset(o, 0, sizeof(double) * (size_t)d_out);
        for (int p = 0; p < n_paths; ++p) {
            const int *q = pt + p * PT_FIELDS;
            int mi = q[PT_MUL_IN], mo = q[PT_MUL_OUT], n3 = q[PT_N3];
            for (int u = 0; u < mi; ++u) {
                for (int k = 0; k < n3; ++k) t[k] = 0.0;
                for (int z = q[PT_NZ0]; z < q[PT_NZ0] + q[PT_NZN]; ++z) {
                    double xv = ld(x, (size_t)r * d_x + q[PT_A] + u * q[PT_N1] + nzi[z], in_f32);
                    double yv = ld(y, (size_t)r * d_sh + q[PT_B] + nzj[z], in_f32);
                    t[nzk[z]] += nzc[z] * xv * yv;
                }
                for (int ww = 0; ww < mo; ++ww) {
                    double wv = ld(w, (size_t)q[PT_WOFF] + (size_t)u * mo + ww, in_f32);
                    for (int k = 0; k < n3; ++k) o[q[PT_O] + ww * n3 + k] += t[k] * wv;
                }
            }
        }
    }
    return 0;
}

/*
 * uvw batched backward: the derivatives of sum(g * out) written as loops.  For every row, path,
 * input channel u and nonzero (i, j, k, c):
 *   gw[k]  = sum_w W_p[u][w] g[row, o + w*n3 + k]
 *   dx[row, a + u*n1 + i] += c * y[row, b + j] * gw[k]
 *   dy[row, b + j]        += c * x[row, a + u*n1 + i] * gw[k]
 *   t[k] (= sum of c * x * y)  then  dW_p[u][w] += sum_k t[k] * g[row, o + w*n3 + k]
 * dx and dy are written for the n_rows rows; dW sums over the rows `wrows` (n_wrows of them), each
 * thread into its own array, the arrays then added in thread order.
 */
int oracle_uvw_backward(int n_paths, const int *pt, const int *nzi, const int *nzj, const int *nzk,
                        const double *nzc, int d_x, int d_sh, int d_out, int64_t weight_numel, int64_t n_rows,
                        const int64_t *rows, int64_t n_wrows, const int64_t *wrows, const void *x, const void *y,
                        const void *w, const void *g, int in_f32, double *dx, double *dy, double *dw,
                        int n_threads)
{
#pragma omp parallel for schedule(dynamic, 4) num_threads(n_threads)
    for (int64_t s = 0; s < n_rows; ++s) {
        const int64_t r = rows[s];
        double *ox = dx + (size_t)s * d_x, *oy = dy + (size_t)s * d_sh;
        double gw[64];
        memset(ox, 0, sizeof(double) * (size_t)d_x);
        memset(oy, 0, sizeof(double) * (size_t)d_sh);
        for (int p = 0; p < n_paths; ++p) {
            const int *q = pt + p * PT_FIELDS;
            int mi = q[PT_MUL_IN], mo = q[PT_MUL_OUT], n3 = q[PT_N3];
            for (int u = 0; u < mi; ++u) {
                for (int k = 0; k < n3; ++k) {
                    gw[k] = 0.0;
                    for (int ww = 0; ww < mo; ++ww)
                        gw[k] += ld(w, (size_t)q[PT_WOFF] + (size_t)u * mo + ww, in_f32) *
                                 ld(g, (size_t)r * d_out + q[PT_O] + ww * n3 + k, in_f32);
                }
                for (int z = q[PT_NZ0]; z < q[PT_NZ0] + q[PT_NZN]; ++z) {
                    double xv = ld(x, (size_t)r * d_x + q[PT_A] + u * q[PT_N1] + nzi[z], in_f32);
                    double yv = ld(y, (size_t)r * d_sh + q[PT_B] + nzj[z], in_f32);
                    ox[q[PT_A] + u * q[PT_N1] + nzi[z]] += nzc[z] * yv * gw[nzk[z]];
                    oy[q[PT_B] + nzj[z]] += nzc[z] * xv * gw[nzk[z]];
                }
            }
        }
    }
    int nt = n_threads > 0 ? n_threads : 1;
    double *part = (double *)calloc((size_t)nt * (size_t)weight_numel, sizeof(double));
    if (!part) return 1;
#pragma omp parallel num_threads(nt)
    {
        double *mine = part + (size_t)omp_get_thread_num() * (size_t)weight_numel;
        double t[64];
#pragma omp for schedule(static)
        for (int64_t s = 0; s < n_wrows; ++s) {
            const int64_t r = wrows[s];
            for (int p = 0; p < n_paths; ++p) {
                const int *q = pt + p * PT_FIELDS;
                int mi = q[PT_MUL_IN], mo = q[PT_MUL_OUT], n3 = q[PT_N3];
                for (int u = 0; u < mi; ++u) {
                    for (int k = 0; k < n3; ++k) t[k] = 0.0;
                    for (int z = q[PT_NZ0]; z < q[PT_NZ0] + q[PT_NZN]; ++z) {
                        double xv = ld(x, (size_t)r * d_x + q[PT_A] + u * q[PT_N1] + nzi[z], in_f32);
                        double yv = ld(y, (size_t)r * d_sh + q[PT_B] + nzj[z], in_f32);
                        t[nzk[z]] += nzc[z] * xv * yv;
                    }
                    for (int ww = 0; ww < mo; ++ww) {
                        double acc = 0.0;
                        for (int k = 0; k < n3; ++k) acc += t[k] * ld(g, (size_t)r * d_out + q[PT_O] + ww * n3 + k, in_f32);
                        mine[(size_t)q[PT_WOFF] + (size_t)u * mo + ww] += acc;
                    }
                }
            }
        }
    }
    for (int64_t i = 0; i < weight_numel; ++i) {
        double acc = 0.0;
        for (int th = 0; th < nt; ++th) acc += part[(size_t)th * (size_t)weight_numel + i];
        dw[i] = acc;
    }
    free(part);
    return 0;
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
