// extern "C" entry points of libcgtp (declared and documented in include/cgtp.h).
// Argument checks happen here, before any HIP call; kernels are launched
// asynchronously on the caller's stream; nothing is allocated on the device.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <string>

#include "plan.h"
#include "static_kernels.h"

struct cgtp_plan {
    cgtp::Plan p;
};

namespace {

thread_local std::string g_last_error;

cgtp_status fail(cgtp_status code, const std::string &msg)
{
    g_last_error = msg;
    return code;
}

template <class F> cgtp_status guarded(F &&f)
{
    try {
        f();
        return CGTP_OK;
    } catch (const cgtp::Error &e) {
        return fail(e.code, e.what());
    } catch (const std::bad_alloc &) {
        return fail(CGTP_ERR_INTERNAL, "host out of memory");
    } catch (const std::exception &e) {
        return fail(CGTP_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(CGTP_ERR_INTERNAL, "unknown failure");
    }
}

void require(bool ok, const std::string &msg)
{
    if (!ok) throw cgtp::Error(CGTP_ERR_INVALID_ARG, msg);
}

void require_ptr(const void *p, const char *name, size_t align)
{
    require(p != nullptr, std::string(name) + " is NULL");
    require(reinterpret_cast<uintptr_t>(p) % align == 0,
            std::string(name) + " is not aligned to " + std::to_string(align) + " bytes");
}

// [a, a+na) and [b, b+nb) in bytes must not overlap
void require_disjoint(const void *a, size_t na, const char *an, const void *b, size_t nb, const char *bn)
{
    if (!a || !b || !na || !nb) return;
    auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    require(x + na <= y || y + nb <= x, std::string(an) + " overlaps " + bn);
}

void check_hip(hipError_t e, const char *what)
{
    if (e != hipSuccess) throw cgtp::Error(CGTP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void launch(hipFunction_t f, int64_t waves, void **args, void *stream, unsigned lds_bytes = 0)
{
    const int64_t blocks = (waves + 3) / 4;
    require(blocks <= INT_MAX, "problem too large for one launch");
    check_hip(hipModuleLaunchKernel(f, (unsigned)blocks, 1, 1, 256, 1, 1, lds_bytes, static_cast<hipStream_t>(stream),
                                    args, nullptr),
              "hipModuleLaunchKernel");
}

size_t elem(const cgtp::Plan &P) { return P.dtype == CGTP_F64 ? 8 : 4; }

// Waves per receiver row in the receiver-owned passes (forward, double backward's receiver
// pass).  A graph with few receivers leaves most of the chip's wave slots (256 CUs x 4 SIMDs x
// the occupancy target) idle once the first rows finish, and its longest row sets the end;
// splitting each row over 2 or 4 waves of one workgroup (edge groups dealt round-robin, parts
// summed in part order through LDS) shortens both.  The split doubles while the launch stays
// under four waves per slot and every part keeps at least 8 edge groups of the mean row
// (measured, 32 channels at 4 waves per SIMD: N = 5,000 with 40 edges per row 116 / 103 /
// 108 us for 1 / 2 / 4 parts, with 160 edges per row 383 / 333 / 317 us; N = 20,000 with 40
// edges per row even).  The choice depends only on N, E and the plan, so a given graph always
// gets the same bits.  Single-task plans only.
struct RowSplit {
    int split = 1;
    unsigned lds = 0;
};

RowSplit row_split(const cgtp::Plan &P, int64_t N, int64_t E, int waves_per_eu)
{
    RowSplit r;
    if (!cgtp::fwd_splittable(P) || N <= 0) return r;
    if (P.fwd_row_split > 0) {
        r.split = P.fwd_row_split;
    } else {
        const int64_t slots = 1024LL * waves_per_eu;
        const double groups = (double)E / (double)N / P.fwd_groups[0].es;  // edge groups per row
        while (r.split < 4 && N * r.split < 4 * slots && groups / (2 * r.split) >= 8) r.split *= 2;
    }
    if (r.split > 1)
        r.lds = (unsigned)((4 - 4 / r.split) * (size_t)cgtp::fwd_group_accs(P, 0) * P.fwd_groups[0].ct * elem(P));
    if (r.lds > 65536) r = RowSplit{};
    return r;
}

void check_graph_sizes(int64_t N, int64_t E)
{
    require(N >= 0 && N < INT_MAX, "N must be in [0, 2^31-1)");
    require(E >= 0 && E < INT_MAX, "E must be in [0, 2^31-1)");
}

// out[0, wn) = sum over nchunks chunks of the partials ws[chunk][wn] (cgtp_reduce_chunks: one
// 16-wave workgroup per 64 elements)
void launch_reduce(hipFunction_t f, int64_t wn, void *ws, long nchunks, void *out, void *stream)
{
    void *args[] = {&ws, &nchunks, &out};
    check_hip(hipModuleLaunchKernel(f, (unsigned)((wn + 63) / 64), 1, 1, 1024, 1, 1, 0, static_cast<hipStream_t>(stream),
                                    args, nullptr),
              "hipModuleLaunchKernel");
}

// Radial forward: the Theta columns of one path group's channel tile are copied to LDS
void check_radial_fwd(const cgtp::Plan &P, int R)
{
    if (!cgtp::radial_fwd_fits(P, R))
        throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "radial forward: R x (paths of a group) x (channels of a tile) Theta "
                                                "elements exceed the 160 KB LDS of a workgroup (" +
                                                    std::to_string(cgtp::radial_fwd_lds_bytes(P, R)) + " bytes)");
}

// Radial backward: chunks of spc consecutive senders, one workgroup and one dTheta partial each
// (at most 1024 chunks)
void radial_chunks(int64_t N, long &spc, long &nchunks)
{
    nchunks = (long)std::min<int64_t>(N, 1024);
    spc = nchunks > 0 ? (long)((N + nchunks - 1) / nchunks) : 1;
    nchunks = nchunks > 0 ? (long)((N + spc - 1) / spc) : 0;
}

// Sender pass of the backward (one launch per path group, in order): dx, dY and (uvu) dW from
// the output gradient g; A is the plan itself or the uvw convolution's unit-weight plan.
void sender_pass(cgtp::Plan &A, int64_t N, int64_t E, const int32_t *t_row_ptr, const int32_t *t_edge,
                 const int32_t *t_dst, const void *x, const void *y, const void *w, const void *g, void *dx, void *dy,
                 void *dw, void *stream, int acc = 0)
{
    const auto &L = cgtp::module_for_current_device(A);
    long nnodes = (long)N;
    // waves per sender: split the sender's edges when the mean out-degree leaves enough
    // edge groups per wave (the dx partials are then summed in a fixed order in LDS)
    for (int grp = 0; grp < (int)A.bwd_groups.size(); ++grp) {
        const double groups = (double)E / (double)N / A.bwd_groups[grp].es;
        int wpr = groups >= 16 ? 4 : groups >= 8 ? 2 : 1;
        if (const char *env = std::getenv("CGTP_BWD_WPR")) wpr = std::max(1, std::min(4, std::atoi(env)));
        // unit-weight plans (the uvw backward's sender pass) take `acc`: add to the outputs
        void *args[] = {&t_row_ptr, &t_edge, &t_dst, &x, &y, &w, &g, &dx, &dy, &dw, &nnodes, &wpr, &grp, &acc};
        check_hip(hipModuleLaunchKernel(L.conv_bwd, (unsigned)N, 1, 1, 64 * wpr, 1, 1, 0,
                                        static_cast<hipStream_t>(stream), args, nullptr),
                  "hipModuleLaunchKernel");
    }
}

// Workspace of the uvw convolution backward: G (N x sum_p mul_in(p) (2 l3 + 1), padded to 256
// bytes), then one dW partial per 16-receiver tile.  Zero for uvu plans.
size_t conv_uvw_workspace(const cgtp::Plan &P, int64_t N, size_t *g_bytes)
{
    if (g_bytes) *g_bytes = 0;
    if (P.mode != CGTP_UVW || N == 0) return 0;
    const size_t es = elem(P);
    const size_t gb = ((size_t)N * cgtp::conv_uvw_g_width(P) * es + 255) / 256 * 256;
    if (g_bytes) *g_bytes = gb;
    return gb + (size_t)((N + 15) / 16) * P.w_numel * es;
}

// Workspace of the uvw radial backward, each part 256-byte aligned: G (as the uvw backward), the
// dTheta partials of every radial channel (R x 16-receiver tiles x weight_numel), the scaled SH
// rows rho[:, r] y of the current channel and that channel's SH-row gradient (E x d_sh each).
struct uvw_radial_parts {
    size_t g = 0, part = 0, ys = 0, t = 0;
};

size_t uvw_radial_workspace(const cgtp::Plan &P, int64_t N, int64_t E, int R, uvw_radial_parts *parts)
{
    if (N == 0) return 0;
    const size_t es = elem(P);
    auto pad = [](size_t b) { return (b + 255) / 256 * 256; };
    size_t gb = 0;
    conv_uvw_workspace(P, N, &gb);
    uvw_radial_parts q;
    q.g = 0;
    q.part = gb;
    q.ys = q.part + pad((size_t)R * ((N + 15) / 16) * P.w_numel * es);
    q.t = q.ys + pad((size_t)E * P.d_sh * es);
    if (parts) *parts = q;
    return q.t + pad((size_t)E * P.d_sh * es);
}

// The uvw radial backward, channel by channel: with ys = rho[:, r] y and G_r = Theta_r^T g,
// dTheta_r is the uvw dW pass on (x, ys); the unit-weight sender pass on (x, ys, G_r) adds channel
// r's share to dx and yields t = d/dys, which the fold turns into dY += rho[:, r] t and
// drho[:, r] = <y, t>.  Channel 0 writes dx and dY, later channels add; dTheta_r is the sum of its
// tile partials in tile order.
void uvw_radial_backward(cgtp::Plan &P, int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col,
                         const int32_t *t_row_ptr, const int32_t *t_edge, const int32_t *t_dst, const void *x,
                         const void *y, int R, const void *rho, const void *theta, const void *grad_out, void *grad_x,
                         void *grad_y, void *grad_rho, void *grad_theta, void *workspace, const uvw_radial_parts &q,
                         void *stream)
{
    const auto &F = cgtp::conv_uvw_backward_for_current_device(P);
    const size_t es = elem(P);
    const bool f64 = P.dtype == CGTP_F64;
    if (N == 0) {
        if (grad_theta) launch_reduce(F.reduce, (int64_t)R * P.w_numel, workspace, 0, grad_theta, stream);
        return;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    void *G = ws + q.g, *ys = ws + q.ys, *t = ws + q.t;
    long nrows = (long)N;
    const unsigned tiles = (unsigned)((N + 15) / 16);
    const unsigned threads = 1024u / (unsigned)P.uvc_rpw;
    const bool need_t = grad_y || grad_rho;
    const int32_t *order = nullptr;
    for (int r = 0; r < R; ++r) {
        const void *th = static_cast<const char *>(theta) + (size_t)r * P.w_numel * es;
        check_hip(cgtp::launch_radial_scale(f64, E, P.d_sh, R, r, y, rho, ys, st), "radial scale");
        if (grad_theta) {
            void *part = ws + q.part + (size_t)r * tiles * P.w_numel * es;
            for (int grp = 0; grp < (int)P.uvc_groups.size(); ++grp) {
                void *args[] = {&row_ptr, &col, &x, &ys, &grad_out, &part, &nrows, &order, &grp};
                check_hip(hipModuleLaunchKernel(F.w, tiles, 1, 1, threads, 1, 1, 0, st, args, nullptr),
                          "hipModuleLaunchKernel");
            }
        }
        if (grad_x || need_t) {
            long nwaves = (long)tiles * (long)cgtp::conv_uvw_g_items(P, nullptr);
            void *gargs[] = {&th, &grad_out, &G, &nrows, &nwaves};
            launch(F.g, nwaves, gargs, stream);
            cgtp::Plan &A = cgtp::conv_uvw_aux_plan(P);
            sender_pass(A, N, E, t_row_ptr, t_edge, t_dst, x, ys, nullptr, G, grad_x, need_t ? t : nullptr, nullptr,
                        stream, r > 0 ? 1 : 0);
            if (need_t)
                check_hip(cgtp::launch_radial_fold(f64, E, P.d_sh, R, r, y, rho, t, grad_y, grad_rho, r > 0 ? 1 : 0, st),
                          "radial fold");
        }
    }
    if (grad_theta)
        for (int r = 0; r < R; ++r)
            launch_reduce(F.reduce, P.w_numel, ws + q.part + (size_t)r * tiles * P.w_numel * es, (long)tiles,
                          static_cast<char *>(grad_theta) + (size_t)r * P.w_numel * es, stream);
}

}  // namespace

extern "C" {

const char *cgtp_last_error(void) { return g_last_error.c_str(); }

cgtp_status cgtp_plan_create(const char *in_irreps, const char *sh_irreps, const char *out_irreps, cgtp_mode mode,
                             cgtp_dtype dtype, cgtp_plan **plan_out)
{
    return guarded([&] {
        require(in_irreps && sh_irreps && out_irreps && plan_out, "NULL argument to cgtp_plan_create");
        *plan_out = nullptr;
        require(mode == CGTP_UVU || mode == CGTP_UVW, "mode must be CGTP_UVU or CGTP_UVW");
        require(dtype == CGTP_F32 || dtype == CGTP_F64, "dtype must be CGTP_F32 or CGTP_F64");
        auto h = std::make_unique<cgtp_plan>();
        cgtp::Plan &P = h->p;
        P.mode = mode;
        P.dtype = dtype;
        P.ins = cgtp::parse_irreps(in_irreps, "input");
        P.sh = cgtp::parse_irreps(sh_irreps, "SH");
        P.out = cgtp::parse_irreps(out_irreps, "output");
        cgtp::build_paths(P);
        cgtp::schedule(P);
        P.source = cgtp::generate_source(P);
        cgtp::compile_module(P);
        if (const char *log = std::getenv("CGTP_LOG"); log && *log && *log != '0') {
            std::fprintf(stderr, "[cgtp] plan: %zu paths, %d nnz, d_x=%d d_sh=%d d_out=%d, module %zu bytes\n",
                         P.paths.size(), P.nnz_total, P.d_x, P.d_sh, P.d_out, P.code.size());
            for (size_t k = 0; k < P.fwd_groups.size(); ++k)
                std::fprintf(stderr, "[cgtp]   fwd group %zu: %zu paths, mul %d, ct %d, tiles %d\n", k,
                             P.fwd_groups[k].paths.size(), P.fwd_groups[k].mul, P.fwd_groups[k].ct,
                             P.fwd_groups[k].tiles);
            for (size_t k = 0; k < P.bwd_groups.size(); ++k)
                std::fprintf(stderr, "[cgtp]   bwd group %zu: %zu paths, mul %d, ct %d, tiles %d, prefetch %d\n", k,
                             P.bwd_groups[k].paths.size(), P.bwd_groups[k].mul, P.bwd_groups[k].ct,
                             P.bwd_groups[k].tiles, (int)P.bwd_groups[k].prefetch);
            for (size_t k = 0; k < P.uvc_groups.size(); ++k)
                std::fprintf(stderr, "[cgtp]   uvw convolution group %zu: %zu paths, mul %d, ct %d, tiles %d, %d receivers "
                             "per wave\n", k, P.uvc_groups[k].paths.size(), P.uvc_groups[k].mul, P.uvc_groups[k].ct,
                             P.uvc_groups[k].tiles, P.uvc_rpw);
            for (size_t k = 0; k < P.dbl_groups.size(); ++k)
                std::fprintf(stderr, "[cgtp]   double-backward sender group %zu: %zu paths, mul %d, ct %d, tiles %d\n", k,
                             P.dbl_groups[k].paths.size(), P.dbl_groups[k].mul, P.dbl_groups[k].ct,
                             P.dbl_groups[k].tiles);
            std::fprintf(stderr, "[cgtp]   waves/SIMD targets: fwd %d, bwd %d, double backward %d / %d\n",
                         P.fwd_waves_per_eu, P.bwd_waves_per_eu, P.dbl_fwd_waves_per_eu, P.dbl_bwd_waves_per_eu);
        }
        *plan_out = h.release();
    });
}

cgtp_status cgtp_plan_destroy(cgtp_plan *plan)
{
    return guarded([&] {
        if (!plan) return;
        cgtp::unload_modules(plan->p);
        delete plan;
    });
}

cgtp_status cgtp_plan_info_get(const cgtp_plan *plan, cgtp_plan_info *info)
{
    return guarded([&] {
        require(plan && info, "NULL argument to cgtp_plan_info_get");
        const cgtp::Plan &P = plan->p;
        info->d_x = P.d_x;
        info->d_sh = P.d_sh;
        info->d_out = P.d_out;
        info->num_paths = (int32_t)P.paths.size();
        info->weight_numel = P.w_numel;
        info->nnz_total = P.nnz_total;
        info->mode = P.mode;
        info->dtype = P.dtype;
        info->fwd_tasks = P.fwd_tasks;
    });
}

cgtp_status cgtp_conv_row_split(const cgtp_plan *plan, int64_t N, int64_t E, int32_t pass, int32_t *split)
{
    return guarded([&] {
        require(plan && split, "NULL argument to cgtp_conv_row_split");
        require(pass == 0 || pass == 1, "pass must be 0 (forward) or 1 (double backward, receiver pass)");
        check_graph_sizes(N, E);
        const cgtp::Plan &P = plan->p;
        *split = P.mode == CGTP_UVU ? row_split(P, N, E, pass == 0 ? P.fwd_waves_per_eu : P.dbl_fwd_waves_per_eu).split
                                    : 1;
    });
}

cgtp_status cgtp_plan_path(const cgtp_plan *plan, int32_t path, cgtp_path_info *info)
{
    return guarded([&] {
        require(plan && info, "NULL argument to cgtp_plan_path");
        require(path >= 0 && path < (int32_t)plan->p.paths.size(), "path index out of range");
        const cgtp::Path &p = plan->p.paths[path];
        info->i1 = p.i1;
        info->i2 = p.i2;
        info->slot = p.slot;
        info->l1 = p.l1;
        info->l2 = p.l2;
        info->l3 = p.l3;
        info->p3 = p.p3;
        info->x_off = p.a;
        info->y_off = p.b;
        info->out_off = p.o;
        info->mul_in = p.mul_in;
        info->mul_out = p.mul_out;
        info->w_off = p.w_off;
        info->nnz = (int32_t)p.nz.size();
    });
}

cgtp_status cgtp_plan_path_coefficients(const cgtp_plan *plan, int32_t path, int32_t cap, int32_t *ijk,
                                        double *values, int32_t *nnz)
{
    return guarded([&] {
        require(plan && nnz, "NULL argument to cgtp_plan_path_coefficients");
        require(path >= 0 && path < (int32_t)plan->p.paths.size(), "path index out of range");
        require(cap >= 0 && (cap == 0 || (ijk && values)), "cap > 0 needs ijk and values");
        const auto &nz = plan->p.paths[path].nz;
        *nnz = (int32_t)nz.size();
        for (int32_t t = 0; t < cap && t < (int32_t)nz.size(); ++t) {
            ijk[3 * t] = nz[t].i;
            ijk[3 * t + 1] = nz[t].j;
            ijk[3 * t + 2] = nz[t].k;
            values[t] = nz[t].c;
        }
    });
}

const char *cgtp_plan_source(const cgtp_plan *plan) { return plan ? plan->p.source.c_str() : ""; }

cgtp_status cgtp_tp_forward(const cgtp_plan *plan, int64_t B, const void *x, const void *y, const void *w,
                            int shared_weights, void *out, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        require(B >= 0 && B < INT_MAX, "B must be in [0, 2^31-1)");
        if (P.mode == CGTP_UVU)
            require(shared_weights == 0, "uvu takes per-row weights: shared_weights must be 0");
        else
            require(shared_weights == 1, "uvw takes shared weights: shared_weights must be 1");
        if (B == 0) return;
        const size_t es = elem(P);
        require_ptr(x, "x", es);
        require_ptr(y, "y", es);
        require_ptr(w, "w", es);
        require_ptr(out, "out", es);
        const size_t nw = (P.mode == CGTP_UVU ? (size_t)B : 1) * P.w_numel * es;
        require_disjoint(out, B * P.d_out * es, "out", x, B * P.d_x * es, "x");
        require_disjoint(out, B * P.d_out * es, "out", y, B * P.d_sh * es, "y");
        require_disjoint(out, B * P.d_out * es, "out", w, nw, "w");
        if (P.mode == CGTP_UVW) {
            const auto &L = cgtp::module_for_current_device(P);
            long nrows = (long)B, nblocks = (long)((B + 15) / 16);
            void *args[] = {&x, &y, &w, &out, &nrows, &nblocks};
            launch(L.tp_uvw, nblocks * (int64_t)P.uvw_groups.size() * cgtp::uvw_out_tiles(P), args, stream);
            return;
        }
        const auto &L = cgtp::module_for_current_device(P);
        int es_max = 1;
        for (const auto &g : P.fwd_groups) es_max = std::max(es_max, g.es);
        int64_t blocks_of_rows = (B + es_max - 1) / es_max;
        int64_t waves = blocks_of_rows * P.fwd_tasks;
        const void *rp = nullptr, *cp = nullptr, *ord = nullptr;
        long nrows = (long)B, nwaves = (long)waves;
        void *args[] = {&rp, &cp, &x, &y, &w, &out, &nrows, &nwaves, &ord};
        launch(L.tp_fwd, waves, args, stream);
    });
}

cgtp_status cgtp_conv_forward(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col,
                              const void *x, const void *y, const void *w, void *out, void *stream)
{
    return cgtp_conv_forward_ordered(plan, N, E, row_ptr, col, nullptr, x, y, w, out, stream);
}

// uvw batched backward: chunks of 16-row blocks whose dW partials the workspace holds
static void uvb_chunks(int64_t B, long &nblocks, long &bpc, long &nchunks)
{
    nblocks = (long)((B + 15) / 16);
    nchunks = std::min<long>(nblocks, 256);
    bpc = nchunks > 0 ? (nblocks + nchunks - 1) / nchunks : 1;
    nchunks = nchunks > 0 ? (nblocks + bpc - 1) / bpc : 0;
}

// uvw batched backward with a multiplicity above 16: the uvw convolution backward on the identity
// graph (row b is the edge from sender b to receiver b), whose one index array 0, 1, ..., B sits
// in the workspace after the convolution's own part (padded to 256 bytes)
static size_t identity_conv_part(const cgtp::Plan &P, int64_t B)
{
    return (conv_uvw_workspace(P, B, nullptr) + 255) / 256 * 256;
}

cgtp_status cgtp_tp_backward_workspace_size(const cgtp_plan *plan, int64_t B, size_t *bytes)
{
    return guarded([&] {
        require(plan != nullptr && bytes != nullptr, "plan and bytes must be non-NULL");
        const cgtp::Plan &P = plan->p;
        require(B >= 0 && B < INT_MAX, "B must be in [0, 2^31-1)");
        *bytes = 0;
        if (P.mode == CGTP_UVW && !P.uvb_ok) {
            *bytes = identity_conv_part(P, B) + (size_t)(B + 1) * 4;
        } else if (P.mode == CGTP_UVW) {
            long nblocks, bpc, nchunks;
            uvb_chunks(B, nblocks, bpc, nchunks);
            *bytes = (size_t)nchunks * P.w_numel * elem(P);
        }
    });
}

cgtp_status cgtp_tp_backward(const cgtp_plan *plan, int64_t B, const void *x, const void *y, const void *w,
                             int shared_weights, const void *grad_out, void *grad_x, void *grad_y, void *grad_w,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        require(B >= 0 && B < INT_MAX, "B must be in [0, 2^31-1)");
        const bool uvw = P.mode == CGTP_UVW;
        if (!uvw)
            require(shared_weights == 0, "uvu takes per-row weights: shared_weights must be 0");
        else
            require(shared_weights == 1, "uvw takes shared weights: shared_weights must be 1");
        if (uvw && !P.uvb_ok && !P.uvc_ok)
            throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "uvw batched backward with a multiplicity above 16 runs the uvw "
                                                    "convolution backward, which this plan cannot: " + P.uvc_why);
        if (!grad_x && !grad_y && !grad_w) return;
        if (uvw && !P.uvb_ok) {
            const size_t part = identity_conv_part(P, B), need = part + (size_t)(B + 1) * 4;
            require_ptr(workspace, "workspace", 256);
            require(workspace_bytes >= need, "workspace too small (see cgtp_tp_backward_workspace_size)");
            int32_t *ids = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + part);
            check_hip(cgtp::launch_iota(B + 1, ids, static_cast<hipStream_t>(stream)), "iota launch");
            const cgtp_status st = cgtp_conv_backward_ws(plan, B, B, ids, ids, nullptr, ids, ids, ids, x, y, w,
                                                         grad_out, grad_x, grad_y, grad_w, workspace, part, stream);
            if (st != CGTP_OK) throw cgtp::Error(st, g_last_error);
            return;
        }
        const size_t es = elem(P);
        if (B == 0) {
            if (uvw && grad_w) {
                // no rows: the shared-weight gradient is zero
                require_ptr(grad_w, "grad_w", es);
                const auto &F = cgtp::uvw_backward_for_current_device(P);
                launch_reduce(F.reduce, P.w_numel, workspace, 0, grad_w, stream);
            }
            return;
        }
        require_ptr(x, "x", es);
        require_ptr(y, "y", es);
        require_ptr(w, "w", es);
        require_ptr(grad_out, "grad_out", es);
        if (grad_x) require_ptr(grad_x, "grad_x", es);
        if (grad_y) require_ptr(grad_y, "grad_y", es);
        if (grad_w) require_ptr(grad_w, "grad_w", es);
        const size_t nw = (uvw ? 1 : (size_t)B) * P.w_numel * es;
        long nblocks, bpc, nchunks;
        uvb_chunks(B, nblocks, bpc, nchunks);
        const size_t ws_need = uvw && grad_w ? (size_t)nchunks * P.w_numel * es : 0;
        if (ws_need) {
            require_ptr(workspace, "workspace", es);
            require(workspace_bytes >= ws_need, "workspace too small (see cgtp_tp_backward_workspace_size)");
        }
        const void *ins[] = {x, y, w, grad_out};
        const size_t inn[] = {B * P.d_x * es, B * P.d_sh * es, nw, B * P.d_out * es};
        const char *inm[] = {"x", "y", "w", "grad_out"};
        void *outs[] = {grad_x, grad_y, grad_w, ws_need ? workspace : nullptr};
        const size_t outn[] = {B * P.d_x * es, B * P.d_sh * es, nw, ws_need};
        const char *outm[] = {"grad_x", "grad_y", "grad_w", "workspace"};
        for (int a = 0; a < 4; ++a) {
            for (int b = 0; b < 4; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
            for (int b = a + 1; b < 4; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
        }
        long nrows = (long)B;
        if (!uvw) {
            const auto &L = cgtp::module_for_current_device(P);
            // one launch per path group, in order (later groups add to blocks an earlier one wrote)
            for (int grp = 0; grp < (int)P.bwd_groups.size(); ++grp) {
                long nb = (long)((B + P.bwd_groups[grp].es - 1) / P.bwd_groups[grp].es);
                void *args[] = {&x, &y, &w, &grad_out, &grad_x, &grad_y, &grad_w, &nrows, &nb, &grp};
                launch(L.tp_bwd, nb, args, stream);
            }
            return;
        }
        const auto &F = cgtp::uvw_backward_for_current_device(P);
        if (grad_x || grad_y) {
            // one workgroup of four waves per 16-row block; the waves share the input blocks
            void *args[] = {&x, &y, &w, &grad_out, &grad_x, &grad_y, &nrows, &nblocks};
            launch(F.xy, nblocks * 4, args, stream);
        }
        if (grad_w) {
            long nwaves = nchunks * (long)P.uvb_w_groups.size();
            void *args[] = {&x, &y, &grad_out, &workspace, &nrows, &nblocks, &bpc, &nchunks, &nwaves};
            launch(F.w, nwaves, args, stream);
            launch_reduce(F.reduce, P.w_numel, workspace, nchunks, grad_w, stream);
        }
    });
}

cgtp_status cgtp_tp_backward_noalloc(const cgtp_plan *plan, int64_t B, const void *x, const void *y, const void *w,
                                     int shared_weights, const void *grad_out, void *grad_x, void *grad_y,
                                     void *grad_w, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        size_t need = 0;
        cgtp_status st = cgtp_tp_backward_workspace_size(plan, B, &need);
        if (st != CGTP_OK) throw cgtp::Error(st, g_last_error);
        if (need > cgtp::kScratchBytes)
            throw cgtp::Error(CGTP_ERR_UNSUPPORTED,
                              "cgtp_tp_backward_noalloc: this batch needs " + std::to_string(need) +
                                  " bytes of workspace, more than the " + std::to_string(cgtp::kScratchBytes) +
                                  " bytes of the library's fixed device scratch (use cgtp_tp_backward with a "
                                  "caller workspace, or a smaller batch)");
        void *ws = nullptr;
        if (need > 0) check_hip(cgtp::scratch_for_current_device(&ws), "hipGetSymbolAddress(scratch)");
        st = cgtp_tp_backward(plan, B, x, y, w, shared_weights, grad_out, grad_x, grad_y, grad_w, ws,
                              need > 0 ? cgtp::kScratchBytes : 0, stream);
        if (st != CGTP_OK) throw cgtp::Error(st, g_last_error);
    });
}

cgtp_status cgtp_graph_order(int64_t N, const int32_t *row_ptr, int32_t *order, void *stream)
{
    return guarded([&] {
        require(N >= 0 && N < INT_MAX, "N must be in [0, 2^31-1)");
        if (N == 0) return;
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(order, "order", 4);
        require_disjoint(order, N * 4, "order", row_ptr, (N + 1) * 4, "row_ptr");
        check_hip(cgtp::launch_degree_order(N, row_ptr, order, static_cast<hipStream_t>(stream)), "order launch");
    });
}

cgtp_status cgtp_conv_forward_ordered(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                      const int32_t *col, const int32_t *order, const void *x, const void *y,
                                      const void *w, void *out, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        const bool uvw = P.mode == CGTP_UVW;
        if (uvw && !P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
        if (N == 0) return;
        const size_t es = elem(P);
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(out, "out", es);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(x, "x", es);
            require_ptr(y, "y", es);
        }
        if (E > 0 || uvw) require_ptr(w, "w", es);
        const size_t no = N * P.d_out * es;
        require_disjoint(out, no, "out", x, N * P.d_x * es, "x");
        require_disjoint(out, no, "out", y, E * P.d_sh * es, "y");
        require_disjoint(out, no, "out", w, (uvw ? 1 : E) * P.w_numel * es, "w");
        require_disjoint(out, no, "out", row_ptr, (N + 1) * 4, "row_ptr");
        require_disjoint(out, no, "out", col, E * 4, "col");
        if (order) {
            require_ptr(order, "order", 4);
            require_disjoint(out, no, "out", order, N * 4, "order");
        }
        const auto &L = cgtp::module_for_current_device(P);
        if (uvw) {
            // one workgroup of 16 / rpw waves per 16 receivers, one launch per path group, in order
            long nrows = (long)N;
            const unsigned tiles = (unsigned)((N + 15) / 16);
            const unsigned threads = 1024u / (unsigned)P.uvc_rpw;
            for (int grp = 0; grp < (int)P.uvc_groups.size(); ++grp) {
                void *args[] = {&row_ptr, &col, &x, &y, &w, &out, &nrows, &order, &grp};
                check_hip(hipModuleLaunchKernel(L.conv_uvw, tiles, 1, 1, threads, 1, 1, 0,
                                                static_cast<hipStream_t>(stream), args, nullptr),
                          "hipModuleLaunchKernel");
            }
            return;
        }
        const RowSplit rs = row_split(P, N, E, P.fwd_waves_per_eu);
        long nrows = (long)N, nwaves = (long)(N * P.fwd_tasks);
        void *args[] = {&row_ptr, &col, &x, &y, &w, &out, &nrows, &nwaves, &order};
        launch(rs.split == 1 ? L.conv_fwd : L.conv_fwd_split[rs.split / 4], nwaves * rs.split, args, stream, rs.lds);
    });
}

cgtp_status cgtp_plan_uvw_backward_prepare(const cgtp_plan *plan)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        if (P.mode != CGTP_UVW || !P.uvb_ok)
            throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "uvw batched backward: uvw plans with multiplicities <= 16");
        cgtp::prepare_uvw_backward(P);
    });
}

const char *cgtp_plan_uvw_backward_source(const cgtp_plan *plan)
{
    if (!plan) return nullptr;
    cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
    std::lock_guard<std::mutex> lock(P.mu);
    return P.uvb.code.empty() ? nullptr : P.uvb.source.c_str();
}

cgtp_status cgtp_plan_radial_prepare(const cgtp_plan *plan, int32_t R)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        require(R >= 1 && R <= 64, "R (radial features per edge) must be in [1, 64]");
        if (P.mode == CGTP_UVW) {
            // uvw: the kernels of the shared-weight uvw convolution module, one launch per channel
            if (!P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
            cgtp::prepare_conv_uvw_backward(P);
            return;
        }
        check_radial_fwd(P, R);
        cgtp::prepare_radial(P, R);
    });
}

const char *cgtp_plan_radial_source(const cgtp_plan *plan, int32_t R)
{
    if (!plan) return nullptr;
    cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
    std::lock_guard<std::mutex> lock(P.mu);
    if (P.mode == CGTP_UVW) return P.ucb.code.empty() ? nullptr : P.ucb.source.c_str();
    auto it = P.radial.find(R);
    return it == P.radial.end() ? nullptr : it->second.source.c_str();
}

cgtp_status cgtp_conv_forward_radial(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                     const int32_t *col, const int32_t *order, const void *x, const void *y, int32_t R,
                                     const void *rho, const void *theta, void *out, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        require(R >= 1 && R <= 64, "R (radial features per edge) must be in [1, 64]");
        const bool uvw = P.mode == CGTP_UVW;
        const size_t es = elem(P);
        if (uvw && !P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
        if (!uvw) check_radial_fwd(P, R);
        if (N == 0) return;
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(out, "out", es);
        require_ptr(theta, "theta", es);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(x, "x", es);
            require_ptr(y, "y", es);
            require_ptr(rho, "rho", es);
        }
        if (order) require_ptr(order, "order", 4);
        const size_t no = N * P.d_out * es;
        require_disjoint(out, no, "out", x, N * P.d_x * es, "x");
        require_disjoint(out, no, "out", y, E * P.d_sh * es, "y");
        require_disjoint(out, no, "out", rho, E * (size_t)R * es, "rho");
        require_disjoint(out, no, "out", theta, (size_t)R * P.w_numel * es, "theta");
        require_disjoint(out, no, "out", row_ptr, (N + 1) * 4, "row_ptr");
        require_disjoint(out, no, "out", col, E * 4, "col");
        require_disjoint(out, no, "out", order, N * 4, "order");
        if (uvw) {
            // channel r: the uvw convolution of (rho[:, r] y) with Theta's row r; channel 0 writes,
            // the others add, each one launch per path group in order
            const auto &F = cgtp::conv_uvw_backward_for_current_device(P);
            long nrows = (long)N;
            const unsigned tiles = (unsigned)((N + 15) / 16);
            const unsigned threads = 1024u / (unsigned)P.uvc_rpw;
            int nrad = R;
            for (int r = 0; r < R; ++r) {
                int acc = r > 0 ? 1 : 0, rr = r;
                const void *th = static_cast<const char *>(theta) + (size_t)r * P.w_numel * es;
                for (int grp = 0; grp < (int)P.uvc_groups.size(); ++grp) {
                    void *args[] = {&row_ptr, &col, &x, &y, &th, &out, &nrows, &order, &grp, &acc, &rho, &nrad, &rr};
                    check_hip(hipModuleLaunchKernel(F.fwd_rad, tiles, 1, 1, threads, 1, 1, 0,
                                                    static_cast<hipStream_t>(stream), args, nullptr),
                              "hipModuleLaunchKernel");
                }
            }
            return;
        }
        hipFunction_t f = cgtp::radial_functions_for_current_device(P, R).fwd;
        // one wave per row: splitting rows measured no faster here (each extra workgroup
        // stages Theta again; N = 5,000, R = 8: 121 / 121 / 140 us for 1 / 2 / 4 parts).
        // Workgroups of 4 receivers, one (path group, channel tile) each: fwd_tasks * ceil(N / 4).
        long nrows = (long)N, nwaves = (long)(P.fwd_tasks * ((N + 3) / 4) * 4);
        void *args[] = {&row_ptr, &col, &x, &y, &rho, &theta, &out, &nrows, &nwaves, &order};
        launch(f, nwaves, args, stream);
    });
}

cgtp_status cgtp_conv_backward_radial_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, int32_t R,
                                                    size_t *bytes)
{
    return guarded([&] {
        require(plan != nullptr && bytes != nullptr, "plan and bytes must be non-NULL");
        check_graph_sizes(N, E);
        require(R >= 1 && R <= 64, "R (radial features per edge) must be in [1, 64]");
        if (plan->p.mode == CGTP_UVW) {
            *bytes = uvw_radial_workspace(plan->p, N, E, R, nullptr);
            return;
        }
        long spc, nchunks;
        radial_chunks(N, spc, nchunks);
        *bytes = (size_t)nchunks * R * plan->p.w_numel * elem(plan->p);
    });
}

cgtp_status cgtp_conv_backward_radial(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                      const int32_t *col, const int32_t *t_row_ptr, const int32_t *t_edge,
                                      const int32_t *t_dst, const void *x, const void *y, int32_t R, const void *rho,
                                      const void *theta, const void *grad_out, void *grad_x, void *grad_y,
                                      void *grad_rho, void *grad_theta, void *workspace, size_t workspace_bytes,
                                      void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        require(R >= 1 && R <= 64, "R (radial features per edge) must be in [1, 64]");
        const bool uvw = P.mode == CGTP_UVW;
        if (uvw && !P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
        const size_t es = elem(P);
        if (!grad_x && !grad_y && !grad_rho && !grad_theta) return;
        const size_t nth = (size_t)R * P.w_numel * es;
        if (grad_theta) require_ptr(grad_theta, "grad_theta", es);
        long spc, nchunks;
        radial_chunks(N, spc, nchunks);
        uvw_radial_parts parts{};
        const size_t ws_need = uvw ? (N > 0 ? uvw_radial_workspace(P, N, E, R, &parts) : 0)
                                   : grad_theta ? (size_t)nchunks * nth : 0;
        if (N > 0) {
            require_ptr(row_ptr, "row_ptr", 4);
            require_ptr(t_row_ptr, "t_row_ptr", 4);
            require_ptr(x, "x", es);
            require_ptr(theta, "theta", es);
            if (E > 0) {
                require_ptr(col, "col", 4);
                require_ptr(t_edge, "t_edge", 4);
                require_ptr(t_dst, "t_dst", 4);
                require_ptr(y, "y", es);
                require_ptr(rho, "rho", es);
                require_ptr(grad_out, "grad_out", es);
            }
            if (grad_x) require_ptr(grad_x, "grad_x", es);
            if (E > 0 && grad_y) require_ptr(grad_y, "grad_y", es);
            if (E > 0 && grad_rho) require_ptr(grad_rho, "grad_rho", es);
            if (ws_need) {
                require_ptr(workspace, "workspace", 256);
                require(workspace_bytes >= ws_need, "workspace too small (see cgtp_conv_backward_radial_workspace_size)");
            }
            const void *ins[] = {x, y, rho, theta, grad_out, row_ptr, col, t_row_ptr, t_edge, t_dst};
            const size_t inn[] = {N * P.d_x * es, E * P.d_sh * es, E * (size_t)R * es, nth, N * P.d_out * es,
                                  (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)E * 4};
            const char *inm[] = {"x", "y", "rho", "theta", "grad_out", "row_ptr", "col", "t_row_ptr", "t_edge", "t_dst"};
            void *outs[] = {grad_x, grad_y, grad_rho, grad_theta, ws_need ? workspace : nullptr};
            const size_t outn[] = {N * P.d_x * es, E * P.d_sh * es, E * (size_t)R * es, nth, ws_need};
            const char *outm[] = {"grad_x", "grad_y", "grad_rho", "grad_theta", "workspace"};
            for (int a = 0; a < 5; ++a) {
                for (int b = 0; b < 10; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
                for (int b = a + 1; b < 5; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
            }
        }
        if (uvw) {
            uvw_radial_backward(P, N, E, row_ptr, col, t_row_ptr, t_edge, t_dst, x, y, R, rho, theta, grad_out,
                                grad_x, grad_y, grad_rho, grad_theta, workspace, parts, stream);
            return;
        }
        const auto &F = cgtp::radial_functions_for_current_device(P, R);
        if (!F.bwd)
            throw cgtp::Error(CGTP_ERR_UNSUPPORTED,
                              "radial backward: a path group's R x mul_in Theta columns and the reduction buffer "
                              "exceed the 160 KB LDS of a workgroup");
        if (N == 0) {
            if (grad_theta) launch_reduce(F.reduce, (int64_t)R * P.w_numel, workspace, 0, grad_theta, stream);
            return;
        }
        const std::vector<cgtp::Group> &groups = cgtp::radial_bwd_groups_of(P, R);
        void *ws = ws_need ? workspace : nullptr;
        long nnodes = (long)N;
        // one launch per path group, in order (later groups add to dx, dY and drho)
        for (int grp = 0; grp < (int)groups.size(); ++grp) {
            const double eg = (double)E / (double)N / groups[grp].es;
            int wpr = eg >= 16 ? 4 : eg >= 8 ? 2 : 1;
            if (const char *env = std::getenv("CGTP_BWD_WPR")) wpr = std::max(1, std::min(4, std::atoi(env)));
            void *args[] = {&t_row_ptr, &t_edge, &t_dst, &x, &y, &rho, &theta, &grad_out, &grad_x, &grad_y, &grad_rho,
                            &ws, &nnodes, &spc, &wpr, &grp};
            check_hip(hipModuleLaunchKernel(F.bwd, (unsigned)nchunks, 1, 1, 64 * wpr, 1, 1, 0,
                                            static_cast<hipStream_t>(stream), args, nullptr),
                      "hipModuleLaunchKernel");
        }
        if (grad_theta) launch_reduce(F.reduce, (int64_t)R * P.w_numel, workspace, nchunks, grad_theta, stream);
    });
}

cgtp_status cgtp_graph_transpose(int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col, int32_t *t_row_ptr,
                                 int32_t *t_edge, int32_t *t_dst, void *stream)
{
    return guarded([&] {
        check_graph_sizes(N, E);
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(t_row_ptr, "t_row_ptr", 4);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(t_edge, "t_edge", 4);
            require_ptr(t_dst, "t_dst", 4);
        }
        const void *outs[3] = {t_row_ptr, t_edge, t_dst};
        const size_t outn[3] = {(size_t)(N + 1) * 4, (size_t)E * 4, (size_t)E * 4};
        const char *names[3] = {"t_row_ptr", "t_edge", "t_dst"};
        for (int a = 0; a < 3; ++a) {
            require_disjoint(outs[a], outn[a], names[a], row_ptr, (N + 1) * 4, "row_ptr");
            require_disjoint(outs[a], outn[a], names[a], col, E * 4, "col");
            for (int b = a + 1; b < 3; ++b) require_disjoint(outs[a], outn[a], names[a], outs[b], outn[b], names[b]);
        }
        check_hip(cgtp::launch_transpose(N, E, row_ptr, col, t_row_ptr, t_edge, t_dst, static_cast<hipStream_t>(stream)),
                  "transpose launch");
    });
}

cgtp_status cgtp_conv_backward(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col,
                               const int32_t *t_row_ptr, const int32_t *t_edge, const int32_t *t_dst, const void *x,
                               const void *y, const void *w, const void *grad_out, void *grad_x, void *grad_y,
                               void *grad_w, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        if (P.mode != CGTP_UVU) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "uvw convolution backward: use cgtp_conv_backward_ws (it needs a workspace)");
        if (N == 0) return;
        if (!grad_x && !grad_y && !grad_w) return;
        const size_t es = elem(P);
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(t_row_ptr, "t_row_ptr", 4);
        require_ptr(x, "x", es);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(t_edge, "t_edge", 4);
            require_ptr(t_dst, "t_dst", 4);
            require_ptr(y, "y", es);
            require_ptr(w, "w", es);
            require_ptr(grad_out, "grad_out", es);
        }
        if (grad_x) require_ptr(grad_x, "grad_x", es);
        if (E > 0 && grad_y) require_ptr(grad_y, "grad_y", es);
        if (E > 0 && grad_w) require_ptr(grad_w, "grad_w", es);
        const void *ins[] = {x, y, w, grad_out, row_ptr, col, t_row_ptr, t_edge, t_dst};
        const size_t inn[] = {N * P.d_x * es, E * P.d_sh * es, E * P.w_numel * es, N * P.d_out * es,
                              (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)E * 4};
        const char *inm[] = {"x", "y", "w", "grad_out", "row_ptr", "col", "t_row_ptr", "t_edge", "t_dst"};
        void *outs[] = {grad_x, grad_y, grad_w};
        const size_t outn[] = {N * P.d_x * es, E * P.d_sh * es, E * P.w_numel * es};
        const char *outm[] = {"grad_x", "grad_y", "grad_w"};
        for (int a = 0; a < 3; ++a) {
            for (int b = 0; b < 9; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
            for (int b = a + 1; b < 3; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
        }
        // with E == 0 the kernel still runs: every sender has an empty row and writes zeros to grad_x
        sender_pass(P, N, E, t_row_ptr, t_edge, t_dst, x, y, w, grad_out, grad_x, grad_y, grad_w, stream);
    });
}

// Backward in receiver order: edges per wave (a multiple of the widest group's edge slots) and
// the edges of one range [e_lo, e_hi) whose dx contributions fit the workspace.
static long rbw_edges_per_wave(const cgtp::Plan &P, long range_edges)
{
    int es = 1;
    for (const cgtp::Group &g : P.rbw_groups) es = std::max(es, g.es);
    long k = (range_edges + 16383) / 16384;  // about 16k waves per launch
    k = std::max<long>(4, std::min<long>(k, 256));
    return (k + es - 1) / es * es;
}

cgtp_status cgtp_conv_backward_receiver_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, size_t *bytes,
                                                       size_t *min_bytes)
{
    return guarded([&] {
        require(plan != nullptr && bytes != nullptr, "plan and bytes must be non-NULL");
        check_graph_sizes(N, E);
        const cgtp::Plan &P = plan->p;
        if (P.mode != CGTP_UVU) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "the receiver-order backward takes uvu plans");
        const size_t row = (size_t)P.d_x * elem(P);
        *bytes = (size_t)E * row;
        if (min_bytes) *min_bytes = E > 0 ? (size_t)rbw_edges_per_wave(P, E) * row : 0;
    });
}

cgtp_status cgtp_conv_backward_receiver(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                        const int32_t *col, const int32_t *t_row_ptr, const int32_t *t_edge,
                                        const void *x, const void *y, const void *w, const void *grad_out,
                                        void *grad_x, void *grad_y, void *grad_w, void *workspace,
                                        size_t workspace_bytes, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        if (P.mode != CGTP_UVU) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "the receiver-order backward takes uvu plans");
        check_graph_sizes(N, E);
        if (!grad_x && !grad_y && !grad_w) return;
        if (N == 0) return;
        const size_t es = elem(P);
        const size_t row = (size_t)P.d_x * es;
        require_ptr(row_ptr, "row_ptr", 4);
        if (grad_x) {
            require_ptr(t_row_ptr, "t_row_ptr", 4);
            require_ptr(grad_x, "grad_x", es);
        }
        if (grad_y) require_ptr(grad_y, "grad_y", es);
        if (grad_w) require_ptr(grad_w, "grad_w", es);
        long range = E;
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(x, "x", es);
            require_ptr(y, "y", es);
            require_ptr(w, "w", es);
            require_ptr(grad_out, "grad_out", es);
            if (grad_x) {
                require_ptr(t_edge, "t_edge", 4);
                require_ptr(workspace, "workspace", 256);
                const long kmin = rbw_edges_per_wave(P, E);
                require(workspace_bytes >= (size_t)kmin * row,
                        "workspace too small: it must hold the dx rows of at least " + std::to_string(kmin) +
                            " edges (see cgtp_conv_backward_receiver_workspace_size)");
                range = (long)std::min<size_t>((size_t)E, workspace_bytes / row);
            }
        }
        const size_t nx = N * P.d_x * es, ny = E * P.d_sh * es, nw = E * (size_t)P.w_numel * es;
        const size_t wsn = grad_x && E > 0 ? (size_t)range * row : 0;
        const void *ins[] = {x, y, w, grad_out, row_ptr, col, t_row_ptr, t_edge};
        const size_t inn[] = {E > 0 ? nx : 0, ny, nw, E > 0 ? N * P.d_out * es : 0, (size_t)(N + 1) * 4, (size_t)E * 4,
                              grad_x ? (size_t)(N + 1) * 4 : 0, grad_x ? (size_t)E * 4 : 0};
        const char *inm[] = {"x", "y", "w", "grad_out", "row_ptr", "col", "t_row_ptr", "t_edge"};
        void *outs[] = {grad_x, grad_y, grad_w, wsn ? workspace : nullptr};
        const size_t outn[] = {nx, ny, nw, wsn};
        const char *outm[] = {"grad_x", "grad_y", "grad_w", "workspace"};
        for (int a = 0; a < 4; ++a) {
            for (int b = 0; b < 8; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
            for (int b = a + 1; b < 4; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
        }
        const auto &L = cgtp::module_for_current_device(P);
        long nrows = (long)N;
        void *hb = grad_x ? workspace : nullptr;
        if (E == 0) {
            // no edges: dx is zero (the sum over an empty range, written by the first range)
            long e_lo = 0, e_hi = 0;
            int first = 1;
            void *args[] = {&t_row_ptr, &t_edge, &hb, &grad_x, &nrows, &e_lo, &e_hi, &first};
            if (grad_x) launch(L.rbw_dx, nrows, args, stream);
            return;
        }
        for (long e_lo = 0; e_lo < E; e_lo += range) {
            long e_hi = std::min<long>(E, e_lo + range);
            long kper = rbw_edges_per_wave(P, e_hi - e_lo);
            long nwaves = (e_hi - e_lo + kper - 1) / kper;
            for (int grp = 0; grp < (int)P.rbw_groups.size(); ++grp) {
                void *args[] = {&row_ptr, &col, &x, &y, &w, &grad_out, &grad_y, &grad_w, &hb,
                                &nrows, &e_lo, &e_hi, &kper, &grp};
                launch(L.rbw, nwaves, args, stream);
            }
            if (grad_x) {
                int first = e_lo == 0 ? 1 : 0;
                void *args[] = {&t_row_ptr, &t_edge, &hb, &grad_x, &nrows, &e_lo, &e_hi, &first};
                launch(L.rbw_dx, nrows, args, stream);
            }
        }
    });
}

cgtp_status cgtp_conv_backward_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, size_t *bytes)
{
    return guarded([&] {
        require(plan != nullptr && bytes != nullptr, "plan and bytes must be non-NULL");
        check_graph_sizes(N, E);
        *bytes = conv_uvw_workspace(plan->p, N, nullptr);
    });
}

cgtp_status cgtp_conv_backward_ws(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                  const int32_t *col, const int32_t *order, const int32_t *t_row_ptr,
                                  const int32_t *t_edge, const int32_t *t_dst, const void *x, const void *y,
                                  const void *w, const void *grad_out, void *grad_x, void *grad_y, void *grad_w,
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        if (P.mode == CGTP_UVU) {
            const cgtp_status st = cgtp_conv_backward(plan, N, E, row_ptr, col, t_row_ptr, t_edge, t_dst, x, y, w,
                                                      grad_out, grad_x, grad_y, grad_w, stream);
            if (st != CGTP_OK) throw cgtp::Error(st, g_last_error);
            return;
        }
        if (!P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
        if (!grad_x && !grad_y && !grad_w) return;
        const size_t es = elem(P);
        if (grad_w) require_ptr(grad_w, "grad_w", es);
        if (N == 0) {
            // no receivers: dW is zero (grad_x and grad_y are empty)
            if (grad_w) {
                const auto &F = cgtp::conv_uvw_backward_for_current_device(P);
                launch_reduce(F.reduce, P.w_numel, workspace, 0, grad_w, stream);
            }
            return;
        }
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(t_row_ptr, "t_row_ptr", 4);
        require_ptr(x, "x", es);
        require_ptr(w, "w", es);
        require_ptr(grad_out, "grad_out", es);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(t_edge, "t_edge", 4);
            require_ptr(t_dst, "t_dst", 4);
            require_ptr(y, "y", es);
        }
        if (grad_x) require_ptr(grad_x, "grad_x", es);
        if (E > 0 && grad_y) require_ptr(grad_y, "grad_y", es);
        if (order) require_ptr(order, "order", 4);
        size_t g_bytes = 0;
        const size_t ws_need = conv_uvw_workspace(P, N, &g_bytes);
        require_ptr(workspace, "workspace", 256);
        require(workspace_bytes >= ws_need, "workspace too small (see cgtp_conv_backward_workspace_size)");
        const void *ins[] = {x, y, w, grad_out, row_ptr, col, t_row_ptr, t_edge, t_dst, order};
        const size_t inn[] = {N * P.d_x * es, E * P.d_sh * es, P.w_numel * es, N * P.d_out * es,
                              (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)(N + 1) * 4, (size_t)E * 4,
                              (size_t)E * 4, order ? (size_t)N * 4 : 0};
        const char *inm[] = {"x", "y", "w", "grad_out", "row_ptr", "col", "t_row_ptr", "t_edge", "t_dst", "order"};
        void *outs[] = {grad_x, grad_y, grad_w, workspace};
        const size_t outn[] = {N * P.d_x * es, E * P.d_sh * es, P.w_numel * es, ws_need};
        const char *outm[] = {"grad_x", "grad_y", "grad_w", "workspace"};
        for (int a = 0; a < 4; ++a) {
            for (int b = 0; b < 10; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
            for (int b = a + 1; b < 4; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
        }
        const auto &F = cgtp::conv_uvw_backward_for_current_device(P);
        long nrows = (long)N;
        void *G = workspace;
        if (grad_x || grad_y) {
            // G_p = W_p^T g per receiver, then the sender pass of the unit-weight internal plan
            long nwaves = (long)((N + 15) / 16) * (long)cgtp::conv_uvw_g_items(P, nullptr);
            void *args[] = {&w, &grad_out, &G, &nrows, &nwaves};
            launch(F.g, nwaves, args, stream);
            cgtp::Plan &A = cgtp::conv_uvw_aux_plan(P);
            sender_pass(A, N, E, t_row_ptr, t_edge, t_dst, x, y, nullptr, G, grad_x, grad_y, nullptr, stream);
        }
        if (grad_w) {
            // per-tile partials of dW (one launch per path group), summed in tile order
            void *part = static_cast<char *>(workspace) + g_bytes;
            const unsigned tiles = (unsigned)((N + 15) / 16);
            const unsigned threads = 1024u / (unsigned)P.uvc_rpw;
            for (int grp = 0; grp < (int)P.uvc_groups.size(); ++grp) {
                void *args[] = {&row_ptr, &col, &x, &y, &grad_out, &part, &nrows, &order, &grp};
                check_hip(hipModuleLaunchKernel(F.w, tiles, 1, 1, threads, 1, 1, 0, static_cast<hipStream_t>(stream),
                                                args, nullptr),
                          "hipModuleLaunchKernel");
            }
            launch_reduce(F.reduce, P.w_numel, part, (long)tiles, grad_w, stream);
        }
    });
}

cgtp_status cgtp_plan_conv_uvw_backward_prepare(const cgtp_plan *plan)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        if (P.mode != CGTP_UVW) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "uvw convolution backward: uvw plans only");
        if (!P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
        cgtp::prepare_conv_uvw_backward(P);
    });
}

const char *cgtp_plan_conv_uvw_backward_source(const cgtp_plan *plan, int32_t module)
{
    if (!plan || (module != 0 && module != 1)) return nullptr;
    cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
    std::lock_guard<std::mutex> lock(P.mu);
    if (P.ucb.code.empty() || !P.aux) return nullptr;
    return module == 0 ? P.ucb.source.c_str() : P.aux->source.c_str();
}

cgtp_status cgtp_conv_double_backward(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                      const int32_t *col, const int32_t *order, const int32_t *t_row_ptr,
                                      const int32_t *t_edge, const int32_t *t_dst, const void *x, const void *y,
                                      const void *w, const void *grad_out, const void *gg_x, const void *gg_y,
                                      const void *gg_w, void *grad_x, void *grad_y, void *grad_w,
                                      void *grad_grad_out, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        if (P.mode != CGTP_UVU)
            throw cgtp::Error(CGTP_ERR_UNSUPPORTED, "double backward of uvw plans: use cgtp_conv_double_backward_ws "
                                                    "(it needs a workspace)");
        if (N == 0) return;
        const bool send = grad_x || grad_y || grad_w;
        if (!send && !grad_grad_out) return;
        const size_t es = elem(P);
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(x, "x", es);
        require_ptr(gg_x, "gg_x", es);
        if (send) require_ptr(t_row_ptr, "t_row_ptr", 4);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(y, "y", es);
            require_ptr(w, "w", es);
            require_ptr(gg_y, "gg_y", es);
            require_ptr(gg_w, "gg_w", es);
            if (send) {
                require_ptr(t_edge, "t_edge", 4);
                require_ptr(t_dst, "t_dst", 4);
                require_ptr(grad_out, "grad_out", es);
            }
        }
        if (order) require_ptr(order, "order", 4);
        if (grad_x) require_ptr(grad_x, "grad_x", es);
        if (E > 0 && grad_y) require_ptr(grad_y, "grad_y", es);
        if (E > 0 && grad_w) require_ptr(grad_w, "grad_w", es);
        if (grad_grad_out) require_ptr(grad_grad_out, "grad_grad_out", es);
        const void *ins[] = {x, y, w, grad_out, gg_x, gg_y, gg_w, row_ptr, col, order, t_row_ptr, t_edge, t_dst};
        const size_t inn[] = {N * P.d_x * es, E * P.d_sh * es, E * P.w_numel * es, N * P.d_out * es,
                              N * P.d_x * es, E * P.d_sh * es, E * P.w_numel * es, (size_t)(N + 1) * 4,
                              (size_t)E * 4, (size_t)N * 4, (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)E * 4};
        const char *inm[] = {"x", "y", "w", "grad_out", "gg_x", "gg_y", "gg_w", "row_ptr", "col", "order",
                             "t_row_ptr", "t_edge", "t_dst"};
        void *outs[] = {grad_x, grad_y, grad_w, grad_grad_out};
        const size_t outn[] = {N * P.d_x * es, E * P.d_sh * es, E * P.w_numel * es, N * P.d_out * es};
        const char *outm[] = {"grad_x", "grad_y", "grad_w", "grad_grad_out"};
        for (int a = 0; a < 4; ++a) {
            for (int b = 0; b < 13; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
            for (int b = a + 1; b < 4; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
        }
        const auto &L = cgtp::module_for_current_device(P);
        if (grad_grad_out) {
            // receiver pass: d/dg = conv(gg_x, y, w) + conv(x, gg_y, w) + conv(x, y, gg_w)
            const RowSplit rs = row_split(P, N, E, P.dbl_fwd_waves_per_eu);
            long nrows = (long)N, nwaves = (long)(N * P.fwd_tasks);
            void *args[] = {&row_ptr, &col, &x, &y, &w, &gg_x, &gg_y, &gg_w, &grad_grad_out, &nrows, &nwaves, &order};
            launch(rs.split == 1 ? L.dbwd_recv : L.dbwd_recv_split[rs.split / 4], nwaves * rs.split, args, stream,
                   rs.lds);
        }
        if (send) {
            // sender pass over the transpose: d/dx, d/dy, d/dW (one owner per output row)
            long nnodes = (long)N;
            for (int grp = 0; grp < (int)P.dbl_groups.size(); ++grp) {
                const double groups = (double)E / (double)N / P.dbl_groups[grp].es;
                int wpr = groups >= 16 ? 4 : groups >= 8 ? 2 : 1;
                if (const char *env = std::getenv("CGTP_BWD_WPR")) wpr = std::max(1, std::min(4, std::atoi(env)));
                void *args[] = {&t_row_ptr, &t_edge, &t_dst, &x, &y, &w, &grad_out, &gg_x, &gg_y, &gg_w,
                                &grad_x, &grad_y, &grad_w, &nnodes, &wpr, &grp};
                check_hip(hipModuleLaunchKernel(L.dbwd_send, (unsigned)N, 1, 1, 64 * wpr, 1, 1, 0,
                                                static_cast<hipStream_t>(stream), args, nullptr),
                          "hipModuleLaunchKernel");
            }
        }
    });
}

// Workspace of the uvw double backward: G = W^T g and G' = ggw^T g (each N x sum_p mul_in (2 l3 + 1),
// padded to 256 bytes), then two dW partials per 16-receiver tile.  Zero for uvu plans.
static size_t conv_uvw_dbl_workspace(const cgtp::Plan &P, int64_t N, size_t *g_bytes)
{
    size_t gb = 0;
    const size_t one = conv_uvw_workspace(P, N, &gb);
    if (g_bytes) *g_bytes = gb;
    return one == 0 ? 0 : 2 * one;
}

cgtp_status cgtp_conv_double_backward_workspace_size(const cgtp_plan *plan, int64_t N, int64_t E, size_t *bytes)
{
    return guarded([&] {
        require(plan != nullptr && bytes != nullptr, "plan and bytes must be non-NULL");
        check_graph_sizes(N, E);
        *bytes = conv_uvw_dbl_workspace(plan->p, N, nullptr);
    });
}

cgtp_status cgtp_conv_double_backward_ws(const cgtp_plan *plan, int64_t N, int64_t E, const int32_t *row_ptr,
                                         const int32_t *col, const int32_t *order, const int32_t *t_row_ptr,
                                         const int32_t *t_edge, const int32_t *t_dst, const void *x, const void *y,
                                         const void *w, const void *grad_out, const void *gg_x, const void *gg_y,
                                         const void *gg_w, void *grad_x, void *grad_y, void *grad_w,
                                         void *grad_grad_out, void *workspace, size_t workspace_bytes, void *stream)
{
    return guarded([&] {
        require(plan != nullptr, "plan is NULL");
        cgtp::Plan &P = const_cast<cgtp_plan *>(plan)->p;
        check_graph_sizes(N, E);
        if (P.mode == CGTP_UVU) {
            const cgtp_status st = cgtp_conv_double_backward(plan, N, E, row_ptr, col, order, t_row_ptr, t_edge, t_dst, x,
                                                             y, w, grad_out, gg_x, gg_y, gg_w, grad_x, grad_y, grad_w,
                                                             grad_grad_out, stream);
            if (st != CGTP_OK) throw cgtp::Error(st, g_last_error);
            return;
        }
        if (!P.uvc_ok) throw cgtp::Error(CGTP_ERR_UNSUPPORTED, P.uvc_why);
        if (!grad_x && !grad_y && !grad_w && !grad_grad_out) return;
        const size_t es = elem(P);
        if (grad_w) require_ptr(grad_w, "grad_w", es);
        if (N == 0) {
            // no receivers: d/dW is zero (every other result is empty)
            if (grad_w) {
                const auto &F = cgtp::conv_uvw_backward_for_current_device(P);
                launch_reduce(F.reduce, P.w_numel, workspace, 0, grad_w, stream);
            }
            return;
        }
        require_ptr(row_ptr, "row_ptr", 4);
        require_ptr(x, "x", es);
        require_ptr(gg_x, "gg_x", es);
        require_ptr(w, "w", es);
        require_ptr(gg_w, "gg_w", es);
        require_ptr(grad_out, "grad_out", es);
        if (grad_x || grad_y) require_ptr(t_row_ptr, "t_row_ptr", 4);
        if (E > 0) {
            require_ptr(col, "col", 4);
            require_ptr(y, "y", es);
            require_ptr(gg_y, "gg_y", es);
            if (grad_x || grad_y) {
                require_ptr(t_edge, "t_edge", 4);
                require_ptr(t_dst, "t_dst", 4);
            }
        }
        if (grad_x) require_ptr(grad_x, "grad_x", es);
        if (E > 0 && grad_y) require_ptr(grad_y, "grad_y", es);
        if (grad_grad_out) require_ptr(grad_grad_out, "grad_grad_out", es);
        if (order) require_ptr(order, "order", 4);
        size_t g_bytes = 0;
        const size_t ws_need = conv_uvw_dbl_workspace(P, N, &g_bytes);
        const bool need_ws = grad_x || grad_y || grad_w;
        if (need_ws) {
            require_ptr(workspace, "workspace", 256);
            require(workspace_bytes >= ws_need, "workspace too small (see cgtp_conv_double_backward_workspace_size)");
        }
        const size_t nx = N * P.d_x * es, ny = E * P.d_sh * es, nw = P.w_numel * es, no = N * P.d_out * es;
        const void *ins[] = {x, y, w, grad_out, gg_x, gg_y, gg_w, row_ptr, col, t_row_ptr, t_edge, t_dst, order};
        const size_t inn[] = {nx, ny, nw, no, nx, ny, nw, (size_t)(N + 1) * 4, (size_t)E * 4, (size_t)(N + 1) * 4,
                              (size_t)E * 4, (size_t)E * 4, order ? (size_t)N * 4 : 0};
        const char *inm[] = {"x", "y", "w", "grad_out", "gg_x", "gg_y", "gg_w", "row_ptr", "col", "t_row_ptr", "t_edge",
                             "t_dst", "order"};
        void *outs[] = {grad_x, grad_y, grad_w, grad_grad_out, need_ws ? workspace : nullptr};
        const size_t outn[] = {nx, ny, nw, no, ws_need};
        const char *outm[] = {"grad_x", "grad_y", "grad_w", "grad_grad_out", "workspace"};
        for (int a = 0; a < 5; ++a) {
            for (int b = 0; b < 13; ++b) require_disjoint(outs[a], outn[a], outm[a], ins[b], inn[b], inm[b]);
            for (int b = a + 1; b < 5; ++b) require_disjoint(outs[a], outn[a], outm[a], outs[b], outn[b], outm[b]);
        }
        const auto &F = cgtp::conv_uvw_backward_for_current_device(P);
        long nrows = (long)N;
        const unsigned tiles = (unsigned)((N + 15) / 16);
        const unsigned threads = 1024u / (unsigned)P.uvc_rpw;
        if (grad_x || grad_y) {
            // G = W^T g and G' = ggw^T g per receiver; d/dx = dx(ggy, G) + dx(y, G') and d/dy =
            // dY(ggx, G) + dY(x, G'): the unit-weight sender pass twice, the second adding
            void *G0 = workspace;
            void *G1 = static_cast<char *>(workspace) + g_bytes;
            long nwaves = (long)((N + 15) / 16) * (long)cgtp::conv_uvw_g_items(P, nullptr);
            void *a0[] = {&w, &grad_out, &G0, &nrows, &nwaves};
            launch(F.g, nwaves, a0, stream);
            void *a1[] = {&gg_w, &grad_out, &G1, &nrows, &nwaves};
            launch(F.g, nwaves, a1, stream);
            cgtp::Plan &A = cgtp::conv_uvw_aux_plan(P);
            sender_pass(A, N, E, t_row_ptr, t_edge, t_dst, gg_x, gg_y, nullptr, G0, grad_x, grad_y, nullptr, stream, 0);
            sender_pass(A, N, E, t_row_ptr, t_edge, t_dst, x, y, nullptr, G1, grad_x, grad_y, nullptr, stream, 1);
        }
        if (grad_w) {
            // d/dW = dW(T of (ggx, y)) + dW(T of (x, ggy)): the dW pass twice into consecutive
            // per-tile partials, summed in order
            void *part0 = static_cast<char *>(workspace) + 2 * g_bytes;
            void *part1 = static_cast<char *>(part0) + (size_t)tiles * P.w_numel * es;
            const void *xs[2] = {gg_x, x}, *ys[2] = {y, gg_y};
            void *parts[2] = {part0, part1};
            for (int r = 0; r < 2; ++r)
                for (int grp = 0; grp < (int)P.uvc_groups.size(); ++grp) {
                    void *args[] = {&row_ptr, &col, &xs[r], &ys[r], &grad_out, &parts[r], &nrows, &order, &grp};
                    check_hip(hipModuleLaunchKernel(F.w, tiles, 1, 1, threads, 1, 1, 0,
                                                    static_cast<hipStream_t>(stream), args, nullptr),
                              "hipModuleLaunchKernel");
                }
            launch_reduce(F.reduce, P.w_numel, part0, 2 * (long)tiles, grad_w, stream);
        }
        if (grad_grad_out) {
            // d/dg = conv(ggx, y, W) + conv(x, ggy, W) + conv(x, y, ggw): the forward three times,
            // the later ones adding
            const void *xs[3] = {gg_x, x, x}, *ys[3] = {y, gg_y, y}, *ws3[3] = {w, w, gg_w};
            for (int r = 0; r < 3; ++r) {
                int acc = r > 0 ? 1 : 0;
                for (int grp = 0; grp < (int)P.uvc_groups.size(); ++grp) {
                    void *args[] = {&row_ptr, &col, &xs[r], &ys[r], &ws3[r], &grad_grad_out, &nrows, &order, &grp, &acc};
                    check_hip(hipModuleLaunchKernel(F.fwd_acc, tiles, 1, 1, threads, 1, 1, 0,
                                                    static_cast<hipStream_t>(stream), args, nullptr),
                              "hipModuleLaunchKernel");
                }
            }
        }
    });
}

cgtp_status cgtp_spherical_harmonics(int32_t lmax, cgtp_dtype dtype, int64_t E, const void *vec, void *y, void *stream)
{
    return guarded([&] {
        require(lmax >= 0 && lmax <= 7, "lmax must be in [0, 7]");
        require(dtype == CGTP_F32 || dtype == CGTP_F64, "dtype must be CGTP_F32 or CGTP_F64");
        require(E >= 0 && E < INT_MAX, "E must be in [0, 2^31-1)");
        if (E == 0) return;
        const size_t es = dtype == CGTP_F64 ? 8 : 4;
        require_ptr(vec, "vec", es);
        require_ptr(y, "y", es);
        require_disjoint(y, E * (lmax + 1) * (lmax + 1) * es, "y", vec, E * 3 * es, "vec");
        check_hip(cgtp::launch_spherical_harmonics(lmax, dtype == CGTP_F64, E, vec, y, static_cast<hipStream_t>(stream)),
                  "spherical harmonics launch");
    });
}

}  // extern "C"
