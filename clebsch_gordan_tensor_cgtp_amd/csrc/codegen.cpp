// HIP source generator of libcgtp: one gfx950 module per plan, with the real
// CG nonzeros written into the code as literal constants.
//
// Design sources: sciencestack.ai page (TL;DR, Abstract): JIT generation,
// register-resident subkernels with long arithmetic streams, fusion of the
// tensor product with the graph convolution; "The GPU memory optimization
// with Larger angular momentum" discussion: nonzeros in the instruction
// stream, no temporary device memory; Sobek page (Abstract): edge-local
// products consumed directly into bounded receiver-side state; LunaTP page
// (Abstract): node-centric execution with path-group parallelism.
//
// Kernels (all 64-lane wavefronts, 256-thread workgroups of independent waves):
//  cgtp_conv_fwd  one wave per (receiver, path group, channel tile); lanes are
//                 channels; when a group has fewer than 64 channels the wave
//                 works on 64/ct edges at once (edge slots) and sums the slots
//                 at the end.  Accumulators stay in registers across the
//                 receiver's CSR row; each output element is written once.
//                 A launch may give each receiver `split` consecutive waves of
//                 one workgroup (edge groups dealt round-robin); the parts are
//                 summed through LDS in part order.
//  cgtp_conv_bwd  one wave per sender over the sender-sorted transpose; every
//                 path in one wave.  Per edge it forms B_ij = sum_k C_ijk g_k,
//                 then dF/dx_i = sum_j B_ij y_j and dF/dy_j = sum_i B_ij x_i,
//                 writes dW once, reduces dY over the channel lanes, and keeps
//                 dx in registers.  Channel tiles beyond 64 are walked in
//                 sequence by the same wave; dY of later tiles is added to the
//                 value the same lane wrote before, so the sum order is fixed.
//  cgtp_tp_fwd    batched rows (use case A), same arithmetic as the forward.
#include <algorithm>
#include <cstdio>
#include <map>
#include <set>
#include <sstream>

#include "plan.h"

namespace cgtp {

namespace {

struct Out {
    std::ostringstream s;
    int ind = 0;
    template <class... A> Out &operator()(const A &...a)
    {
        for (int i = 0; i < ind; ++i) s << "  ";
        (s << ... << a);
        s << "\n";
        return *this;
    }
};

std::string lit(double v, bool f64)
{
    char buf[64];
    if (f64)
        std::snprintf(buf, sizeof buf, "%a", v);
    else
        std::snprintf(buf, sizeof buf, "%af", (double)(float)v);  // round to nearest float
    return buf;
}

int log2i(int v)
{
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Input blocks, SH blocks and output slots touched by a set of paths.
struct Touch {
    std::set<int> i1, i2, slots;
};
Touch touched(const Plan &P, const std::vector<int> &paths)
{
    Touch t;
    for (int i : paths) {
        t.i1.insert(P.paths[i].i1);
        t.i2.insert(P.paths[i].i2);
        t.slots.insert(P.paths[i].slot);
    }
    return t;
}

int n_of(int l) { return 2 * l + 1; }

// v += v(lane ^ m): the permlane exchange for m = 16, 32, a lane shuffle below
std::string xadd(const std::string &v, int m)
{
    if (m == 16 || m == 32) return v + " = xsum" + std::to_string(m) + "(" + v + ");";
    return v + " += __shfl_xor(" + v + ", " + std::to_string(m) + ");";
}

// (i1, i2) pairs in order of their first path, each with its paths.
std::vector<std::pair<std::pair<int, int>, std::vector<int>>> pairs_of(const Plan &P, const std::vector<int> &paths)
{
    std::vector<std::pair<std::pair<int, int>, std::vector<int>>> out;
    std::map<std::pair<int, int>, int> at;
    for (int i : paths) {
        auto key = std::make_pair(P.paths[i].i1, P.paths[i].i2);
        auto it = at.find(key);
        if (it == at.end()) {
            at[key] = (int)out.size();
            out.push_back({key, {i}});
        } else {
            out[it->second].second.push_back(i);
        }
    }
    return out;
}

// Is lane channel u possibly >= mul (masked) for a block of multiplicity mul?
bool needs_mask(int mul, const Group &g) { return mul != g.tiles * g.ct; }



// Emit loads of the sender row (x), the edge row (y) and the weights of edge index `ei`
// and sender `si` into registers named <pre>x.., <pre>y.., <pre>w..
void emit_edge_loads(Out &o, const Plan &P, const Group &g, const Touch &t, const std::string &pre,
                     const std::string &si, const std::string &ei, bool declare, bool dbl = false, int radial = 0)
{
    const std::string T = declare ? "T " : "";
    for (int b : t.i1) {
        const Irrep &ir = P.ins[b];
        int off = 0;
        for (int pi : g.paths)
            if (P.paths[pi].i1 == b) off = P.paths[pi].a;
        bool m = needs_mask(ir.mul, g);
        for (int i = 0; i < n_of(ir.l); ++i) {
            std::ostringstream addr;
            addr << "x[(size_t)" << si << " * DX + " << off << " + u * " << n_of(ir.l) << " + " << i << "]";
            if (m)
                o(T, pre, "x", b, "_", i, " = (u < ", ir.mul, ") ? ", addr.str(), " : (T)0;");
            else
                o(T, pre, "x", b, "_", i, " = ", addr.str(), ";");
        }
    }
    for (int b : t.i2) {
        int off = 0;
        for (int pi : g.paths)
            if (P.paths[pi].i2 == b) off = P.paths[pi].b;
        for (int j = 0; j < n_of(P.sh[b].l); ++j)
            o(T, pre, "y", b, "_", j, " = LD_STREAM(&y[(size_t)", ei, " * DSH + ", off + j, "]);");
    }
    if (radial) {
        // radial features of the edge (the weights are rebuilt from them, see emit_radial_weights)
        for (int r = 0; r < radial; ++r) o(T, pre, "rho", r, " = LD_STREAM(&rho[(size_t)", ei, " * NRAD + ", r, "]);");
        return;
    }
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        std::ostringstream addr;
        addr << "LD_STREAM(&w[(size_t)" << ei << " * WROW + " << p.w_off << " + u])";
        if (needs_mask(p.mul_in, g))
            o(T, pre, "w", pi, " = (u < ", p.mul_in, ") ? ", addr.str(), " : (T)0;");
        else
            o(T, pre, "w", pi, " = ", addr.str(), ";");
    }
    if (!dbl) return;
    // double backward: the upstream gradients for dx (gathered like x), dY and dW
    for (int b : t.i1) {
        const Irrep &ir = P.ins[b];
        int off = 0;
        for (int pi : g.paths)
            if (P.paths[pi].i1 == b) off = P.paths[pi].a;
        bool m = needs_mask(ir.mul, g);
        for (int i = 0; i < n_of(ir.l); ++i) {
            std::ostringstream addr;
            addr << "ggx[(size_t)" << si << " * DX + " << off << " + u * " << n_of(ir.l) << " + " << i << "]";
            if (m)
                o(T, pre, "gx", b, "_", i, " = (u < ", ir.mul, ") ? ", addr.str(), " : (T)0;");
            else
                o(T, pre, "gx", b, "_", i, " = ", addr.str(), ";");
        }
    }
    for (int b : t.i2) {
        int off = 0;
        for (int pi : g.paths)
            if (P.paths[pi].i2 == b) off = P.paths[pi].b;
        for (int j = 0; j < n_of(P.sh[b].l); ++j)
            o(T, pre, "gy", b, "_", j, " = LD_STREAM(&ggy[(size_t)", ei, " * DSH + ", off + j, "]);");
    }
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        std::ostringstream addr;
        addr << "LD_STREAM(&ggw[(size_t)" << ei << " * WROW + " << p.w_off << " + u])";
        if (needs_mask(p.mul_in, g))
            o(T, pre, "gw", pi, " = (u < ", p.mul_in, ") ? ", addr.str(), " : (T)0;");
        else
            o(T, pre, "gw", pi, " = ", addr.str(), ";");
    }
}

void emit_copy(Out &o, const Plan &P, const Group &g, const Touch &t, const std::string &dst, const std::string &src,
               bool dbl = false, int radial = 0)
{
    for (int b : t.i1)
        for (int i = 0; i < n_of(P.ins[b].l); ++i) o(dst, "x", b, "_", i, " = ", src, "x", b, "_", i, ";");
    for (int b : t.i2)
        for (int j = 0; j < n_of(P.sh[b].l); ++j) o(dst, "y", b, "_", j, " = ", src, "y", b, "_", j, ";");
    if (radial) {
        for (int r = 0; r < radial; ++r) o(dst, "rho", r, " = ", src, "rho", r, ";");
        return;
    }
    for (int pi : g.paths) o(dst, "w", pi, " = ", src, "w", pi, ";");
    if (!dbl) return;
    for (int b : t.i1)
        for (int i = 0; i < n_of(P.ins[b].l); ++i) o(dst, "gx", b, "_", i, " = ", src, "gx", b, "_", i, ";");
    for (int b : t.i2)
        for (int j = 0; j < n_of(P.sh[b].l); ++j) o(dst, "gy", b, "_", j, " = ", src, "gy", b, "_", j, ";");
    for (int pi : g.paths) o(dst, "gw", pi, " = ", src, "gw", pi, ";");
}

// sum_n c_n * <prefix><k_n> over the nonzeros in v (the B_ij = sum_k C_ijk g_k of the backward)
std::string cg_sum_k(const std::vector<const Nonzero *> &v, const std::string &prefix, bool f64)
{
    std::ostringstream e;
    e << lit(v[0]->c, f64) << " * " << prefix << v[0]->k;
    for (size_t n = 1; n < v.size(); ++n) {
        std::ostringstream f;
        f << "FMA(" << lit(v[n]->c, f64) << ", " << prefix << v[n]->k << ", " << e.str() << ")";
        e.str(f.str());
    }
    return e.str();
}

// Linear combination sum_n c_n * <reg prefix><i>_<j> of the nonzeros in v, as nested FMAs.
std::string cg_sum(const std::vector<const Nonzero *> &v, const std::string &reg, bool f64)
{
    std::ostringstream e;
    e << lit(v[0]->c, f64) << " * " << reg << v[0]->i << "_" << v[0]->j;
    for (size_t n = 1; n < v.size(); ++n) {
        std::ostringstream f;
        f << "FMA(" << lit(v[n]->c, f64) << ", " << reg << v[n]->i << "_" << v[n]->j << ", " << e.str() << ")";
        e.str(f.str());
    }
    return e.str();
}

// Double backward, receiver pass: d/dg of <ggx,dx> + <ggy,dy> + <ggw,dW> is the
// convolution of (ggx, y, W) + (x, ggy, W) + (x, y, ggw), so per path and k
//   acc[k] += w * sum C (ggx_i y_j + x_i ggy_j) + ggw * sum C x_i y_j.
void emit_dbl_recv_math(Out &o, const Plan &P, const Group &g, bool f64, const std::string &pre)
{
    for (auto &pr : pairs_of(P, g.paths)) {
        int i1 = pr.first.first, i2 = pr.first.second;
        std::set<std::pair<int, int>> used;
        for (int pi : pr.second)
            for (const Nonzero &z : P.paths[pi].nz) used.insert({z.i, z.j});
        o("{");
        o.ind++;
        for (auto &ij : used) {
            const int i = ij.first, j = ij.second;
            o("const T q", i, "_", j, " = ", pre, "x", i1, "_", i, " * ", pre, "y", i2, "_", j, ";");
            o("const T r", i, "_", j, " = FMA(", pre, "x", i1, "_", i, ", ", pre, "gy", i2, "_", j, ", ", pre, "gx", i1,
              "_", i, " * ", pre, "y", i2, "_", j, ");");
        }
        for (int pi : pr.second) {
            const Path &p = P.paths[pi];
            std::map<int, std::vector<const Nonzero *>> byk;
            for (const Nonzero &z : p.nz) byk[z.k].push_back(&z);
            for (auto &kv : byk)
                o("a", p.slot, "_", kv.first, " = FMA(", pre, "w", pi, ", ", cg_sum(kv.second, "r", f64), ", FMA(", pre,
                  "gw", pi, ", ", cg_sum(kv.second, "q", f64), ", a", p.slot, "_", kv.first, "));");
        }
        o.ind--;
        o("}");
    }
}

// Radial projection (Sobek page, Abstract: reassociated radial projection): the edge's weights
// W[p][u] = sum_r rho_r Theta[r][w_p + u] are rebuilt in registers from the R radial features
// and an LDS copy of the Theta columns the launch unit reads, never stored.  The copy is compact,
// [r][col] with the unit's paths side by side: a forward workgroup holds one channel tile of one
// path group (ct columns per path, zero past the path's channels), a backward workgroup one whole
// path group (mul_in columns per path).  Consecutive lanes read consecutive words.
long theta_width(const Plan &P, const Group &g, bool per_tile)
{
    long w = 0;
    for (int pi : g.paths) w += per_tile ? g.ct : P.paths[pi].mul_in;
    return w;
}

// LDS index of Theta[r][w_p + u] in the unit's copy; `uu` is the (masked) channel
std::string theta_index(const Plan &P, const Group &g, int pi, int r, bool per_tile, const std::string &uu)
{
    long off = 0;
    for (int q : g.paths) {
        if (q == pi) break;
        off += per_tile ? g.ct : P.paths[q].mul_in;
    }
    const std::string col = per_tile ? "(lane & " + std::to_string(g.ct - 1) + ")" : uu;
    return std::to_string((long)r * theta_width(P, g, per_tile) + off) + " + " + col;
}

// The workgroup copies the unit's Theta columns into `thl` (a barrier must follow); the forward
// form needs `tile` in scope
void emit_theta_stage(Out &o, const Plan &P, const Group &g, int R, bool per_tile, const std::string &nthreads)
{
    const long width = theta_width(P, g, per_tile);
    long off = 0;
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        const int n = per_tile ? g.ct : p.mul_in;
        o("for (int i = threadIdx.x; i < ", (long)R * n, "; i += ", nthreads, ") {");
        o.ind++;
        o("const int r = i / ", n, ", c = i - r * ", n, ";");
        if (per_tile && needs_mask(p.mul_in, g)) {
            o("const int uu = tile * ", g.ct, " + c;");
            o("thl[r * ", width, " + ", off, " + c] = uu < ", p.mul_in, " ? theta[(size_t)r * WROW + ", p.w_off,
              " + uu] : (T)0;");
        } else if (per_tile) {
            o("thl[r * ", width, " + ", off, " + c] = theta[(size_t)r * WROW + ", p.w_off, " + tile * ", g.ct, " + c];");
        } else {
            o("thl[r * ", width, " + ", off, " + c] = theta[(size_t)r * WROW + ", p.w_off, " + c];");
        }
        o.ind--;
        o("}");
        off += n;
    }
}

void emit_radial_weights(Out &o, const Plan &P, const Group &g, const std::string &pre, int R, int only, bool per_tile)
{
    for (int pi : g.paths) {
        if (only >= 0 && pi != only) continue;
        const Path &p = P.paths[pi];
        const bool m = needs_mask(p.mul_in, g);
        // lanes past the block read an in-bounds column and their weight is set to 0
        const std::string uu = m ? "(u < " + std::to_string(p.mul_in) + " ? u : 0)" : "u";
        std::ostringstream e;
        e << pre << "rho0 * th[" << theta_index(P, g, pi, 0, per_tile, uu) << "]";
        for (int r = 1; r < R; ++r) {
            std::ostringstream f;
            f << "FMA(" << pre << "rho" << r << ", th[" << theta_index(P, g, pi, r, per_tile, uu) << "], " << e.str()
              << ")";
            e.str(f.str());
        }
        if (m)
            o("const T ", pre, "w", pi, " = (u < ", p.mul_in, ") ? ", e.str(), " : (T)0;");
        else
            o("const T ", pre, "w", pi, " = ", e.str(), ";");
    }
}

// acc[slot][k] += w_p * sum_{ij} C_ijk x_i y_j for every path of the group (radial > 0: each
// path's weight is rebuilt from the radial features right before its use).
void emit_forward_math(Out &o, const Plan &P, const Group &g, bool f64, const std::string &pre, int radial = 0)
{
    for (auto &pr : pairs_of(P, g.paths)) {
        int i1 = pr.first.first, i2 = pr.first.second;
        std::set<std::pair<int, int>> used;
        for (int pi : pr.second)
            for (const Nonzero &z : P.paths[pi].nz) used.insert({z.i, z.j});
        o("{");
        o.ind++;
        for (auto &ij : used)
            o("const T q", ij.first, "_", ij.second, " = ", pre, "x", i1, "_", ij.first, " * ", pre, "y", i2, "_",
              ij.second, ";");
        for (int pi : pr.second) {
            const Path &p = P.paths[pi];
            if (radial) emit_radial_weights(o, P, g, pre, radial, pi, true);
            std::map<int, std::vector<const Nonzero *>> byk;
            for (const Nonzero &z : p.nz) byk[z.k].push_back(&z);
            for (auto &kv : byk) {
                const auto &v = kv.second;
                std::ostringstream e;
                e << lit(v[0]->c, f64) << " * q" << v[0]->i << "_" << v[0]->j;
                for (size_t n = 1; n < v.size(); ++n) {
                    std::ostringstream f;
                    f << "FMA(" << lit(v[n]->c, f64) << ", q" << v[n]->i << "_" << v[n]->j << ", " << e.str() << ")";
                    e.str(f.str());
                }
                o("a", p.slot, "_", kv.first, " = FMA(", pre, "w", pi, ", ", e.str(), ", a", p.slot, "_", kv.first,
                  ");");
            }
        }
        o.ind--;
        o("}");
    }
}

void emit_preamble(Out &o, const Plan &P)
{
    const bool f64 = P.dtype == CGTP_F64;
    o("// generated by libcgtp for in=", P.ins.size(), " irreps, sh=", P.sh.size(), " irreps, out=", P.out.size(),
      " irreps, ", P.paths.size(), " paths, ", P.nnz_total, " CG nonzeros");
    o("typedef ", f64 ? "double" : "float", " T;");
    o("#define FMA(a, b, c) ", f64 ? "__builtin_fma(a, b, c)" : "__builtin_fmaf(a, b, c)");
    o("#define DX ", P.d_x);
    o("#define DSH ", P.d_sh);
    o("#define DOUT ", P.d_out);
    o("#define WROW ", P.w_numel, "L");
    o("typedef unsigned long size_t;");
    // The wave's index in its workgroup, read from the first lane: the compiler then knows it is
    // the same in every lane, so the receiver/sender/edge indices derived from it live in SGPRs
    // and their row_ptr, col and y reads become scalar loads (fewer VGPRs, no per-lane address
    // arithmetic).
    if (P.scalar_wave)
        o("#define WAVE_IN_BLOCK() ((int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6))");
    else
        o("#define WAVE_IN_BLOCK() ((int)(threadIdx.x >> 6))");
    // v(l) + v(l ^ 16) and v(l) + v(l ^ 32) in every lane l.  A v_permlane16_swap of v with itself
    // returns two registers holding the 16-lane rows (0, 0, 2, 2) and (1, 1, 3, 3) of v, a
    // v_permlane32_swap the halves (lo, lo) and (hi, hi); the sum of the two is the xor butterfly's
    // value bit for bit (IEEE addition commutes), from a VALU exchange instead of the LDS round
    // trip of a lane shuffle
    if (P.permlane_sums) {
        for (int m : {16, 32}) {
            o("__device__ __forceinline__ T xsum", m, "(T v)");
            o("{");
            o.ind++;
            // the two results are copied into plain variables first: bit-casting the builtin's
            // vector elements directly made the front end read element 0 for both
            if (f64) {
                o("const unsigned long long b = __builtin_bit_cast(unsigned long long, v);");
                o("const auto lo = __builtin_amdgcn_permlane", m, "_swap((unsigned)b, (unsigned)b, false, false);");
                o("const auto hi = __builtin_amdgcn_permlane", m, "_swap((unsigned)(b >> 32), (unsigned)(b >> 32), false, false);");
                o("const unsigned l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];");
                o("return __builtin_bit_cast(double, ((unsigned long long)h0 << 32) | l0) + "
                  "__builtin_bit_cast(double, ((unsigned long long)h1 << 32) | l1);");
            } else {
                o("const unsigned a = __builtin_bit_cast(unsigned, v);");
                o("const auto r = __builtin_amdgcn_permlane", m, "_swap(a, a, false, false);");
                o("const unsigned r0 = r[0], r1 = r[1];");
                o("return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);");
            }
            o.ind--;
            o("}");
        }
    } else {
        o("#define xsum16(v) ((v) + __shfl_xor((v), 16))");
        o("#define xsum32(v) ((v) + __shfl_xor((v), 32))");
    }
    // per-edge rows read or written once (y, W, dW): streaming hint on the memory instructions
    if (P.stream_hint) {
        o("#define LD_STREAM(p) __builtin_nontemporal_load(p)");
        o("#define ST_STREAM(v, p) __builtin_nontemporal_store(v, p)");
    } else {
        o("#define LD_STREAM(p) (*(p))");
        o("#define ST_STREAM(v, p) (*(p) = (v))");
    }
    o("");
}

// Forward body of one group; `n` is the receiver (conv) or the row block (rows
// mode).  With dbl, the same receiver-owned stream computes the double
// backward's d/dg (emit_dbl_recv_math) from the extra operands ggx, ggy, ggw.
// The parts of a split receiver row, summed in part order through LDS.  The part waves of one
// receiver are consecutive waves of the workgroup, and every wave of the workgroup reaches the
// barrier (split is uniform over the launch).
void emit_part_sum(Out &o, const Plan &P, int gi, const Touch &t)
{
    const Group &g = P.fwd_groups[gi];
    const long span = (long)fwd_group_accs(P, gi) * g.ct;
    o("if constexpr (SPLIT > 1) {");
    o.ind++;
    o("T* red = pred + (long)((threadIdx.x >> 6) / SPLIT) * (SPLIT - 1) * ", span, " + (lane & ", g.ct - 1, ");");
    o("if (part != 0 && slot == 0) {");
    o.ind++;
    o("T* r = red + (long)(part - 1) * ", span, ";");
    int i = 0;
    for (int q : t.slots)
        for (int k = 0; k < n_of(P.out[q].l); ++k, ++i) o("r[", (long)i * g.ct, "] = a", q, "_", k, ";");
    o.ind--;
    o("}");
    o("__syncthreads();");
    o("if (part == 0 && slot == 0) {");
    o.ind++;
    o("for (int p = 1; p < SPLIT; ++p) {");
    o.ind++;
    o("const T* r = red + (long)(p - 1) * ", span, ";");
    i = 0;
    for (int q : t.slots)
        for (int k = 0; k < n_of(P.out[q].l); ++k, ++i) o("a", q, "_", k, " += r[", (long)i * g.ct, "];");
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    o.ind--;
    o("}");
}

void emit_fwd_group(Out &o, const Plan &P, int gi, bool rows, bool dbl = false, int radial = 0)
{
    const Group &g = P.fwd_groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    Touch t = touched(P, g.paths);
    if (!rows && fwd_splittable(P)) o("template <int SPLIT>  // waves per receiver row");
    o("__device__ __forceinline__ void ", rows ? "tp" : dbl ? "dbr" : radial ? "rad" : "fwd", "_g", gi,
      "(long n, int tile, int lane, const int* __restrict__ row_ptr, const int* __restrict__ col, "
      "const T* __restrict__ x, const T* __restrict__ y, ",
      radial ? "const T* __restrict__ rho, const T* thl, " : "const T* __restrict__ w, ",
      dbl ? "const T* __restrict__ ggx, const T* __restrict__ ggy, const T* __restrict__ ggw, " : "",
      "T* __restrict__ out, long nrows", rows ? "" : ", int part, bool live, T* pred", ")");
    o("{");
    o.ind++;
    o("const int slot = lane >> ", log2i(g.ct), ";");
    o("const int u = tile * ", g.ct, " + (lane & ", g.ct - 1, ");");
    if (rows) {
        int es_max = 1;
        for (const Group &h : P.fwd_groups) es_max = std::max(es_max, h.es);
        o("for (int sub = 0; sub < ", es_max / g.es, "; ++sub) {");
        o.ind++;
    }
    for (int q : t.slots)
        for (int k = 0; k < n_of(P.out[q].l); ++k) o("T a", q, "_", k, " = (T)0;");
    if (rows) {
        int es_max = 1;
        for (const Group &h : P.fwd_groups) es_max = std::max(es_max, h.es);
        o("const long r = n * ", es_max, " + sub * ", g.es, " + slot;");
        o("if (r < nrows) {");
        o.ind++;
        emit_edge_loads(o, P, g, t, "c", "r", "r", true);
        emit_forward_math(o, P, g, f64, "c");
        o.ind--;
        o("}");
        o("if (r < nrows) {");
        o.ind++;
        o("T* orow = out + (size_t)r * DOUT;");
    } else {
        // `split` waves share the receiver's row: part p takes edge groups p, p + split, ...
        const bool splittable = fwd_splittable(P);
        if (splittable) {
            o("const int e0 = row_ptr[n], e1 = live ? row_ptr[n + 1] : e0;");
            o("constexpr int stride = SPLIT * ", g.es, ";");
        } else {
            o("const int e0 = row_ptr[n], e1 = row_ptr[n + 1];");
            o("constexpr int stride = ", g.es, ";");
        }
        o("if (e0 < e1) {");
        o.ind++;
        // pipeline: senders (col) two edge groups ahead, operands one ahead, so
        // every wait is for loads issued a whole iteration earlier
        o("int e = e0 + part * ", g.es, " + slot;");
        o("int ec = e < e1 ? e : e1 - 1;");
        o("int s = col[ec];");
        o("int en = (e + stride < e1) ? e + stride : e1 - 1;");
        o("int sn = col[en];");
        emit_edge_loads(o, P, g, t, "c", "s", "ec", true, dbl, radial);
        // keep the next edge's loads ahead of this edge's arithmetic: left alone the scheduler
        // sinks them to the end of the iteration (fewer live registers), and each edge then waits
        // for its own operands
        auto barrier = [&]() {
            if (P.fwd_sched_barrier)
                o("__builtin_amdgcn_sched_barrier(0);");
            else if (splittable && !dbl && !radial && P.split_sched_barrier)
                // rows split over several waves only where receivers are few against the wave
                // slots: there the few resident waves cannot hide each edge's wait, and the pinned
                // loads pay
                o("if constexpr (SPLIT > 1) __builtin_amdgcn_sched_barrier(0);");
        };
        auto math = [&](const std::string &pre) {
            if (radial) {
                // The Theta reads do not depend on the edge: left alone, the compiler hoists all
                // R * paths of them out of the loop and spills them.  An empty asm makes the base
                // offset (always 0) opaque per iteration, so each read stays next to its use.
                o("{");
                o.ind++;
                o("int zo = 0;");
                o("asm volatile(\"\" : \"+v\"(zo));");
                o("const T* th = thl + zo;");
                emit_forward_math(o, P, g, f64, pre, radial);
                o.ind--;
                o("}");
            } else if (dbl) {
                emit_dbl_recv_math(o, P, g, f64, pre);
            } else {
                emit_forward_math(o, P, g, f64, pre);
            }
        };
        if (P.fwd_unroll > 1) {
            // two edges per iteration, the operand sets alternating: the first half computes on
            // the c set and loads the n set, the second computes on n and reloads c, so no operand
            // is copied from one set to the other
            o("for (; e < e1; e += 2 * stride) {");
            o.ind++;
            o("const int enn = (e + 2 * stride < e1) ? e + 2 * stride : e1 - 1;");
            o("const int snn = col[enn];");
            emit_edge_loads(o, P, g, t, "n", "sn", "en", true, dbl, radial);
            barrier();
            math("c");
            o("if (e + stride >= e1) break;");
            o("const int e3 = (e + 3 * stride < e1) ? e + 3 * stride : e1 - 1;");
            o("const int s3 = col[e3];");
            emit_edge_loads(o, P, g, t, "c", "snn", "enn", false, dbl, radial);
            barrier();
            math("n");
            o("en = e3;");
            o("sn = s3;");
            o.ind--;
            o("}");
        } else {
            o("for (; e < e1; e += stride) {");
            o.ind++;
            o("const int enn = (e + 2 * stride < e1) ? e + 2 * stride : e1 - 1;");
            o("const int snn = col[enn];");
            emit_edge_loads(o, P, g, t, "n", "sn", "en", true, dbl, radial);
            barrier();
            math("c");
            emit_copy(o, P, g, t, "c", "n", dbl, radial);
            o("en = enn;");
            o("sn = snn;");
            o.ind--;
            o("}");
        }
        o.ind--;
        o("}");
        // sum the edge slots (fixed butterfly order, identical in every run)
        for (int m = 32; m >= g.ct; m /= 2)
            for (int q : t.slots)
                for (int k = 0; k < n_of(P.out[q].l); ++k) o(xadd("a" + std::to_string(q) + "_" + std::to_string(k), m));
        if (splittable) {
            emit_part_sum(o, P, gi, t);
            o("if (live && part == 0 && slot == 0) {");
        } else {
            o("if (slot == 0) {");
        }
        o.ind++;
        o("T* orow = out + (size_t)n * DOUT;");
    }
    for (int q : t.slots) {
        const Irrep &ir = P.out[q];
        int off = 0;
        for (int pi : g.paths)
            if (P.paths[pi].slot == q) off = P.paths[pi].o;
        std::string guard = needs_mask(ir.mul, g) ? "if (u < " + std::to_string(ir.mul) + ") " : "";
        for (int k = 0; k < n_of(ir.l); ++k)
            o(guard, "orow[", off, " + u * ", n_of(ir.l), " + ", k, "] = a", q, "_", k, ";");
    }
    o.ind--;
    o("}");
    if (rows) {
        o.ind--;
        o("}");  // sub-block loop
    }
    o.ind--;
    o("}");
    o("");
}

// Wave -> (receiver, task, part) of the receiver-owned passes.  `nwaves` counts (receiver, task)
// units.  With split > 1 (single-task plans only) each receiver has `split` consecutive waves of
// one workgroup, and the waves past the last receiver stay alive to the barrier of the part sum
// without touching memory.
void emit_fwd_unit(Out &o, const Plan &P, int split)
{
    if (split == 1) {
        o("T* pred = nullptr;");
        o("if (wave >= nwaves) return;");
        o("const int part = 0;");
        o("const bool live = true;");
        o("const int task = (int)(wave % ", P.fwd_tasks, ");");
        o("long n = wave / ", P.fwd_tasks, ";");
        o("if (order) n = order[n];  // receiver schedule (heavy rows first), results unchanged");
        return;
    }
    o("extern __shared__ T pred[];  // part sums: ", 4 - 4 / split, " waves x accumulators x lanes");
    o("const long unit = wave / ", split, ";");
    o("const int part = (int)(wave % ", split, ");");
    o("const bool live = unit < nwaves;");
    o("const int task = 0;");
    o("long n = live ? unit : 0;");
    o("if (live && order) n = order[n];  // receiver schedule (heavy rows first), results unchanged");
}

// Name suffix of the receiver-owned kernel that gives each row `split` waves.
std::string split_suffix(int split) { return split == 1 ? "" : "_split" + std::to_string(split); }

void emit_fwd_kernel(Out &o, const Plan &P, bool rows, bool dbl = false, int split = 1)
{
    int waves = dbl ? P.dbl_fwd_waves_per_eu : !rows && P.conv_fwd_waves ? P.conv_fwd_waves : P.fwd_waves_per_eu;
    if (!rows && !dbl && split > 1 && P.split_sched_barrier && P.split_fwd_waves) waves = P.split_fwd_waves;
    o("extern \"C\" __global__ void __launch_bounds__(256, ", waves, ") ",
      rows ? "cgtp_tp_fwd" : dbl ? "cgtp_conv_dbwd_recv" : "cgtp_conv_fwd", split_suffix(split),
      "(const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, ",
      dbl ? "const T* __restrict__ ggx, const T* __restrict__ ggy, const T* __restrict__ ggw, " : "",
      "T* __restrict__ out, long nrows, long nwaves, const int* __restrict__ order)");
    o("{");
    o.ind++;
    o("const long wave = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    if (rows) {
        o("if (wave >= nwaves) return;");
        o("const int task = (int)(wave % ", P.fwd_tasks, ");");
        o("long n = wave / ", P.fwd_tasks, ";");
    } else {
        emit_fwd_unit(o, P, split);
    }
    const std::string targ = !rows && fwd_splittable(P) ? "<" + std::to_string(split) + ">" : "";
    o("switch (task) {");
    int task = 0;
    for (int gi = 0; gi < (int)P.fwd_groups.size(); ++gi)
        for (int tile = 0; tile < P.fwd_groups[gi].tiles; ++tile, ++task)
            o("case ", task, ": ", rows ? "tp" : dbl ? "dbr" : "fwd", "_g", gi, targ, "(n, ", tile,
              ", lane, row_ptr, col, x, y, w, ", dbl ? "ggx, ggy, ggw, " : "", "out, nrows",
              rows ? "" : ", part, live, pred", "); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// ------------------------------------------------------------------------------------------
// Backward, sender pass.

// Sum over the CT channel lanes of one edge slot; every lane of the slot ends
// with the same bits (each butterfly step adds the same two operands).
void emit_slot_sum(Out &o, const Plan &P)
{
    const bool f64 = P.dtype == CGTP_F64;
    o("template <int CT> __device__ __forceinline__ T slot_sum(T v)");
    o("{");
    o.ind++;
    const int ctrls[4] = {0xB1, 0x4E, 0x141, 0x140};  // xor1, xor2, half-row mirror, row mirror
    for (int st = 0, m = 2; st < 4; ++st, m *= 2) {
        o("if constexpr (CT >= ", m, ") {");
        o.ind++;
        if (f64) {
            o("long long b = __builtin_bit_cast(long long, v);");
            o("int lo = __builtin_amdgcn_mov_dpp((int)b, ", ctrls[st], ", 15, 15, false);");
            o("int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), ", ctrls[st], ", 15, 15, false);");
            o("v += __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);");
        } else {
            o("v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ", ctrls[st],
              ", 15, 15, false));");
        }
        o.ind--;
        o("}");
    }
    o("if constexpr (CT >= 32) v = xsum16(v);");
    o("if constexpr (CT >= 64) v = xsum32(v);");
    o("return v;");
    o.ind--;
    o("}");
    o("");
}

// Backward, sender pass, one path group (see the file comment).  dx blocks
// and dY blocks are written by the first group that touches them (group 0 also
// writes zeros for blocks no path touches) and accumulated by later groups;
// the groups are separate launches in group order, so the sums are fixed.
// radial backward: dTheta sums reduced over the waves of a workgroup per round (bounds its LDS)
constexpr int kRadialRound = 32;
constexpr long kLdsBytes = 160 * 1024;  // LDS of one gfx950 workgroup

void emit_bwd_group(Out &o, const Plan &P, int gi, bool dbl = false, bool rowmode = false, int radial = 0,
                    const std::vector<Group> *radial_groups = nullptr)
{
    const std::vector<Group> &groups = radial ? *radial_groups : dbl ? P.dbl_groups : P.bwd_groups;
    const Group &g = groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    const bool pf = g.prefetch && !rowmode;
    // Rolling prefetch (first-order pass): an operand's next-edge value is loaded into its register
    // right after the current edge's last use of it (a path's W after that path, a gradient or SH
    // block after the last path reading it), so the next edge's loads stream in while this edge's
    // later paths compute.  Registers are reused rather than doubled, but every operand now lives
    // across the loop's back edge, which raises the count (it pays only for split plans).
    const bool roll = P.bwd_rolling && !pf && !rowmode && !dbl && !radial;
    std::map<int, int> last_of_slot, last_of_i2;  // operand block -> last path (emission order) using it
    for (int pi : g.paths) {
        last_of_slot[P.paths[pi].slot] = pi;
        last_of_i2[P.paths[pi].i2] = pi;
    }
    Touch t = touched(P, g.paths);
    // first group (in launch order) touching each input / SH block
    auto first_i1 = [&](int b) {
        for (int k = 0; k < (int)groups.size(); ++k)
            for (int pi : groups[k].paths)
                if (P.paths[pi].i1 == b) return k;
        return -1;
    };
    auto first_i2 = [&](int b) {
        for (int k = 0; k < (int)groups.size(); ++k)
            for (int pi : groups[k].paths)
                if (P.paths[pi].i2 == b) return k;
        return -1;
    };
    std::vector<int> xb;  // input blocks this group writes or adds
    for (int b = 0; b < (int)P.ins.size(); ++b)
        if (t.i1.count(b) || (gi == 0 && first_i1(b) < 0)) xb.push_back(b);
    int nx = 0;
    for (int b : xb) nx += n_of(P.ins[b].l);
    std::vector<int> yb;  // SH blocks this group writes or adds
    for (int b = 0; b < (int)P.sh.size(); ++b)
        if (t.i2.count(b) || (gi == 0 && first_i2(b) < 0)) yb.push_back(b);

    if (rowmode) {
        // batched rows: edge slot = row; the row is its own sender, edge and receiver
        o("__device__ __forceinline__ void tpb_g", gi,
          "(long blk, int lane, const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ w, "
          "const T* __restrict__ g, T* __restrict__ dx, T* __restrict__ dy, T* __restrict__ dw, long nrows)");
        o("{");
        o.ind++;
        o("const int slot = lane >> ", log2i(g.ct), ";");
        o("const int ul = lane & ", g.ct - 1, ";");
        o("const long row = blk * ", g.es, " + slot;");
        o("const bool live = row < nrows;");
        o("const long s = live ? row : nrows - 1;  // rows past the end read row nrows-1 and store nothing");
    } else if (radial) {
        // radial projection: a chunk of senders [c0, c1) per workgroup; dTheta partials of the
        // chunk accumulate in registers and go to ws[chunk] at the end
        o("__device__ __forceinline__ void rbw_g", gi,
          "(long chunk, long c0, long c1, int wv, int lane, int wpr, T* red, const int* __restrict__ t_row_ptr, "
          "const int* __restrict__ t_edge, const int* __restrict__ t_dst, const T* __restrict__ x, "
          "const T* __restrict__ y, const T* __restrict__ rho, const T* th, const T* __restrict__ g, "
          "T* __restrict__ dx, T* __restrict__ dy, T* __restrict__ drho, T* __restrict__ ws)");
        o("{");
        o.ind++;
        o("const int slot = lane >> ", log2i(g.ct), ";");
        o("const int ul = lane & ", g.ct - 1, ";");
        o("const int stride = ", g.es, " * wpr;");
    } else {
    o("__device__ __forceinline__ void ", dbl ? "dbs" : "bwd", "_g", gi,
      "(long s, int wv, int lane, int wpr, T* red, const int* __restrict__ t_row_ptr, const int* __restrict__ t_edge, "
      "const int* __restrict__ t_dst, const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ w, "
      "const T* __restrict__ g, ",
      dbl ? "const T* __restrict__ ggx, const T* __restrict__ ggy, const T* __restrict__ ggw, " : "",
      "T* __restrict__ dx, T* __restrict__ dy, T* __restrict__ dw", P.unit_weights ? ", int acc" : "", ")");
    o("{");
    o.ind++;
    o("const int slot = lane >> ", log2i(g.ct), ";");
    o("const int ul = lane & ", g.ct - 1, ";");
    o("const int t0 = t_row_ptr[s], t1 = t_row_ptr[s + 1];");
    o("const int stride = ", g.es, " * wpr;");
    }
    o("for (int tile = 0; tile < ", g.tiles, "; ++tile) {");
    o.ind++;
    o("const int u = tile * ", g.ct, " + ul;");
    if (radial) {
        for (int r = 0; r < radial; ++r)
            for (int pi : g.paths) o("T ta", r, "_", pi, " = (T)0;  // dTheta[r][w_p + u] of the chunk");
        o("for (long s = c0; s < c1; ++s) {");
        o.ind++;
        o("const int t0 = t_row_ptr[s], t1 = t_row_ptr[s + 1];");
    }
    for (int b : xb) {
        const Irrep &ir = P.ins[b];
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.ins[bb].dim();
        for (int i = 0; i < n_of(ir.l); ++i) {
            if (t.i1.count(b)) {
                std::string addr = "x[(size_t)s * DX + " + std::to_string(off) + " + u * " + std::to_string(n_of(ir.l)) +
                                   " + " + std::to_string(i) + "]";
                if (needs_mask(ir.mul, g))
                    o("const T x", b, "_", i, " = (u < ", ir.mul, ") ? ", addr, " : (T)0;");
                else
                    o("const T x", b, "_", i, " = ", addr, ";");
                if (dbl) {
                    std::string gaddr = "ggx" + addr.substr(1);
                    if (needs_mask(ir.mul, g))
                        o("const T gx", b, "_", i, " = (u < ", ir.mul, ") ? ", gaddr, " : (T)0;");
                    else
                        o("const T gx", b, "_", i, " = ", gaddr, ";");
                }
            }
            o("T d", b, "_", i, " = (T)0;");
        }
    }
    auto edge_loads = [&](const std::string &pre, const std::string &ev, const std::string &nv, bool declare) {
        const std::string Ty = declare ? "T " : "";
        for (int b : t.i2) {
            int off = 0;
            for (int bb = 0; bb < b; ++bb) off += P.sh[bb].dim();
            for (int j = 0; j < n_of(P.sh[b].l); ++j)
                o(Ty, pre, "y", b, "_", j, " = LD_STREAM(&y[(size_t)", ev, " * DSH + ", off + j, "]);");
        }
        for (int r = 0; r < radial; ++r) o(Ty, pre, "rho", r, " = LD_STREAM(&rho[(size_t)", ev, " * NRAD + ", r, "]);");
        for (int pi : g.paths) {
            if (P.unit_weights || radial) break;
            const Path &p = P.paths[pi];
            std::string wa = "LD_STREAM(&w[(size_t)" + ev + " * WROW + " + std::to_string(p.w_off) + " + u])";
            if (needs_mask(p.mul_in, g))
                o(Ty, pre, "w", pi, " = (u < ", p.mul_in, ") ? ", wa, " : (T)0;");
            else
                o(Ty, pre, "w", pi, " = ", wa, ";");
        }
        for (int q : t.slots) {
            const Irrep &ir = P.out[q];
            int off = 0;
            for (int qq = 0; qq < q; ++qq) off += P.out[qq].dim();
            for (int k = 0; k < n_of(ir.l); ++k) {
                std::string ga = "g[(size_t)" + nv + " * DOUT + " + std::to_string(off) + " + u * " +
                                 std::to_string(n_of(ir.l)) + " + " + std::to_string(k) + "]";
                if (needs_mask(ir.mul, g))
                    o(Ty, pre, "g", q, "_", k, " = (u < ", ir.mul, ") ? ", ga, " : (T)0;");
                else
                    o(Ty, pre, "g", q, "_", k, " = ", ga, ";");
            }
        }
        if (!dbl) return;
        for (int b : t.i2) {
            int off = 0;
            for (int bb = 0; bb < b; ++bb) off += P.sh[bb].dim();
            for (int j = 0; j < n_of(P.sh[b].l); ++j)
                o(Ty, pre, "gy", b, "_", j, " = LD_STREAM(&ggy[(size_t)", ev, " * DSH + ", off + j, "]);");
        }
        for (int pi : g.paths) {
            const Path &p = P.paths[pi];
            std::string wa = "LD_STREAM(&ggw[(size_t)" + ev + " * WROW + " + std::to_string(p.w_off) + " + u])";
            if (needs_mask(p.mul_in, g))
                o(Ty, pre, "gw", pi, " = (u < ", p.mul_in, ") ? ", wa, " : (T)0;");
            else
                o(Ty, pre, "gw", pi, " = ", wa, ";");
        }
    };
    // pipeline: edge and receiver ids two iterations ahead, operands one ahead
    // (with prefetch) so every wait is for loads issued an iteration earlier
    if (rowmode) {
        o("{");
        o.ind++;
        o("{");
        o.ind++;
        o("const long e = s, n = s;");
        edge_loads("", "e", "n", true);
    } else {
    o("int t = t0 + wv * ", g.es, " + slot;");
    o("if (t < t1) {");
    o.ind++;
    o("int e = t_edge[t], n = t_dst[t];");
    o("int tn = (t + stride < t1) ? t + stride : t;");
    o("int en = t_edge[tn], nn = t_dst[tn];");
    if (pf || roll) edge_loads("", "e", "n", true);
    o("for (; t < t1; t += stride) {");
    o.ind++;
    o("const int tnn = (t + 2 * stride < t1) ? t + 2 * stride : tn;");
    o("const int enn = t_edge[tnn], nnn = t_dst[tnn];");
    if (pf)
        edge_loads("n", "en", "nn", true);
    else if (!roll)
        edge_loads("", "e", "n", true);
    }
    for (int b : yb)
        for (int j = 0; j < n_of(P.sh[b].l); ++j) o("T h", b, "_", j, " = (T)0;");  // dF/dy partial of this lane
    for (int r = 0; r < radial; ++r) o("T dr", r, " = (T)0;  // drho[e][r] partial of this lane");
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        // B_ij = sum_k C_ijk g_k
        std::map<std::pair<int, int>, std::vector<const Nonzero *>> byij;
        for (const Nonzero &z : p.nz) byij[{z.i, z.j}].push_back(&z);
        o("{");
        o.ind++;
        if (radial) emit_radial_weights(o, P, g, "", radial, pi, false);
        for (auto &kv : byij) {
            const auto &v = kv.second;
            std::ostringstream e;
            e << lit(v[0]->c, f64) << " * g" << p.slot << "_" << v[0]->k;
            for (size_t n = 1; n < v.size(); ++n) {
                std::ostringstream f;
                f << "FMA(" << lit(v[n]->c, f64) << ", g" << p.slot << "_" << v[n]->k << ", " << e.str() << ")";
                e.str(f.str());
            }
            o("const T B", kv.first.first, "_", kv.first.second, " = ", e.str(), ";");
        }
        // dF/dx_i = sum_j B_ij y_j ; dF/dy_j = sum_i B_ij x_i
        std::map<int, std::vector<int>> rows, cols;
        for (auto &kv : byij) {
            rows[kv.first.first].push_back(kv.first.second);
            cols[kv.first.second].push_back(kv.first.first);
        }
        // f<name>_i = sum_j B_ij <v>_j over the row i (or the column j when by_col)
        auto contract = [&](const std::map<int, std::vector<int>> &lines, bool by_col, const std::string &v, int blk,
                            const std::string &name) {
            for (auto &kv : lines) {
                auto bij = [&](int m) {
                    return by_col ? "B" + std::to_string(m) + "_" + std::to_string(kv.first)
                                  : "B" + std::to_string(kv.first) + "_" + std::to_string(m);
                };
                std::ostringstream e;
                e << bij(kv.second[0]) << " * " << v << blk << "_" << kv.second[0];
                for (size_t n = 1; n < kv.second.size(); ++n) {
                    std::ostringstream f;
                    f << "FMA(" << bij(kv.second[n]) << ", " << v << blk << "_" << kv.second[n] << ", " << e.str() << ")";
                    e.str(f.str());
                }
                o("const T ", name, kv.first, " = ", e.str(), ";");
            }
        };
        // unit weights (the uvw convolution's sender pass): dx_i and dY_j take their terms as one
        // FMA chain each, the running sum innermost (no separate add per row or column)
        auto fold = [&](const std::map<int, std::vector<int>> &lines, bool by_col, const std::string &v, int blk,
                        const std::string &acc) {
            for (auto &kv : lines) {
                std::string e = acc + std::to_string(kv.first);
                for (int m : kv.second) {
                    const std::string b = by_col ? "B" + std::to_string(m) + "_" + std::to_string(kv.first)
                                                 : "B" + std::to_string(kv.first) + "_" + std::to_string(m);
                    e = "FMA(" + b + ", " + v + std::to_string(blk) + "_" + std::to_string(m) + ", " + e + ")";
                }
                o(acc, kv.first, " = ", e, ";");
            }
        };
        const bool folded = P.unit_weights && !dbl && !radial;
        if (folded) {
            fold(rows, false, "y", p.i2, "d" + std::to_string(p.i1) + "_");
            fold(cols, true, "x", p.i1, "h" + std::to_string(p.i2) + "_");
        } else {
            contract(rows, false, "y", p.i2, "fx");
            contract(cols, true, "x", p.i1, "fy");
        }
        if (dbl) contract(rows, false, "gy", p.i2, "fxg");  // d/dx of the ggy term
        if (dbl) contract(cols, true, "gx", p.i1, "fyg");   // d/dy of the ggx term
        if (!P.unit_weights) {
            // dW = sum_i x_i dF/dx_i   (double backward: sum_i ggx_i fx_i + x_i fxg_i)
            std::ostringstream e;
            bool first = true;
            auto term = [&](const std::string &a, const std::string &b) {
                if (first) {
                    e << a << " * " << b;
                    first = false;
                } else {
                    std::ostringstream f;
                    f << "FMA(" << a << ", " << b << ", " << e.str() << ")";
                    e.str(f.str());
                }
            };
            for (auto &kv : rows) {
                const std::string i = std::to_string(kv.first), b1 = std::to_string(p.i1);
                if (dbl) {
                    term("gx" + b1 + "_" + i, "fx" + i);
                    term("x" + b1 + "_" + i, "fxg" + i);
                } else {
                    term("x" + b1 + "_" + i, "fx" + i);
                }
            }
            if (radial) {
                // dW_e[p][u] is consumed at once: drho[e][r] += dW Theta[r][w_p + u] (summed over the
                // lanes below), dTheta[r][w_p + u] += rho[e][r] dW (summed over the chunk's edges)
                const std::string uu = needs_mask(p.mul_in, g) ? "(u < " + std::to_string(p.mul_in) + " ? u : 0)" : "u";
                o("const T dwv = ", e.str(), ";");
                for (int r = 0; r < radial; ++r) {
                    o("dr", r, " = FMA(dwv, th[", theta_index(P, g, pi, r, false, uu), "], dr", r, ");");
                    o("ta", r, "_", pi, " = FMA(rho", r, ", dwv, ta", r, "_", pi, ");");
                }
            } else {
                std::string guard = needs_mask(p.mul_in, g) ? "(u < " + std::to_string(p.mul_in) + ") && " : "";
                if (rowmode) guard = "live && " + guard;
                o("if (", guard, "dw) ST_STREAM(", e.str(), ", &dw[(size_t)e * WROW + ", p.w_off, " + u]);");
            }
        }
        if (dbl) {
            // d/dx = W fxg + ggw fx ; d/dy = W fyg + ggw fy
            for (auto &kv : rows)
                o("d", p.i1, "_", kv.first, " = FMA(w", pi, ", fxg", kv.first, ", FMA(gw", pi, ", fx", kv.first, ", d", p.i1,
                  "_", kv.first, "));");
            for (auto &kv : cols)
                o("h", p.i2, "_", kv.first, " = FMA(w", pi, ", fyg", kv.first, ", FMA(gw", pi, ", fy", kv.first, ", h", p.i2,
                  "_", kv.first, "));");
        } else if (P.unit_weights) {
            if (!folded) {
                for (auto &kv : rows) o("d", p.i1, "_", kv.first, " += fx", kv.first, ";");
                for (auto &kv : cols) o("h", p.i2, "_", kv.first, " += fy", kv.first, ";");
            }
        } else {
            for (auto &kv : rows)
                o("d", p.i1, "_", kv.first, " = FMA(w", pi, ", fx", kv.first, ", d", p.i1, "_", kv.first, ");");
            for (auto &kv : cols)
                o("h", p.i2, "_", kv.first, " = FMA(w", pi, ", fy", kv.first, ", h", p.i2, "_", kv.first, ");");
        }
        if (roll) {
            // this edge is done with these operands: load the next edge's into their registers.
            // Barriers on both sides keep the loads after the last uses (so the registers are
            // reused) and ahead of the next path's work.
            if (P.bwd_rolling > 1) o("__builtin_amdgcn_sched_barrier(0);");
            bool any = false;
            if (!P.unit_weights) {
                std::string wa = "LD_STREAM(&w[(size_t)en * WROW + " + std::to_string(p.w_off) + " + u])";
                if (needs_mask(p.mul_in, g))
                    o("w", pi, " = (u < ", p.mul_in, ") ? ", wa, " : (T)0;");
                else
                    o("w", pi, " = ", wa, ";");
                any = true;
            }
            if (last_of_slot[p.slot] == pi) {
                const Irrep &ir = P.out[p.slot];
                int off = 0;
                for (int qq = 0; qq < p.slot; ++qq) off += P.out[qq].dim();
                for (int k = 0; k < n_of(ir.l); ++k) {
                    std::string ga = "g[(size_t)nn * DOUT + " + std::to_string(off) + " + u * " + std::to_string(n_of(ir.l)) + " + " +
                                     std::to_string(k) + "]";
                    if (needs_mask(ir.mul, g))
                        o("g", p.slot, "_", k, " = (u < ", ir.mul, ") ? ", ga, " : (T)0;");
                    else
                        o("g", p.slot, "_", k, " = ", ga, ";");
                }
                any = true;
            }
            if (last_of_i2[p.i2] == pi) {
                int off = 0;
                for (int bb = 0; bb < p.i2; ++bb) off += P.sh[bb].dim();
                for (int j = 0; j < n_of(P.sh[p.i2].l); ++j)
                    o("y", p.i2, "_", j, " = LD_STREAM(&y[(size_t)en * DSH + ", off + j, "]);");
                any = true;
            }
            if (any && P.bwd_rolling > 1) o("__builtin_amdgcn_sched_barrier(0);");
        }
        o.ind--;
        o("}");
    }
    // dY: sum over the slot's channel lanes; lane (j mod ct) of the slot writes or adds j
    o("if (dy) {");
    o.ind++;
    std::vector<std::pair<int, std::string>> hs;  // (column, register)
    for (int b : yb) {
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.sh[bb].dim();
        for (int jj = 0; jj < n_of(P.sh[b].l); ++jj)
            hs.push_back({off + jj, "h" + std::to_string(b) + "_" + std::to_string(jj)});
    }
    for (auto &h : hs) o(h.second, " = slot_sum<", g.ct, ">(", h.second, ");");
    for (size_t r = 0; r * g.ct < hs.size(); ++r) {
        const size_t lo = r * g.ct, hi = std::min(hs.size(), (r + 1) * g.ct);
        // split the chunk by write/add kind of the block its column belongs to
        for (int add = 0; add < 2; ++add) {
            std::vector<std::pair<size_t, int>> sel;  // (lane, column)
            for (size_t c = lo; c < hi; ++c) {
                int col = hs[c].first;
                int blk = 0, acc = 0;
                for (int b = 0; b < (int)P.sh.size(); ++b) {
                    if (col < acc + P.sh[b].dim()) { blk = b; break; }
                    acc += P.sh[b].dim();
                }
                bool is_add = first_i2(blk) >= 0 && first_i2(blk) < gi;
                if ((int)is_add == add) sel.push_back({c - lo, col});
            }
            if (sel.empty()) continue;
            o("{");
            o.ind++;
            o("T v = (T)0;");
            o("int col = -1;");
            for (auto &sc : sel) o("if (ul == ", sc.first, ") { v = ", hs[lo + sc.first].second, "; col = ", sc.second, "; }");
            o(rowmode ? "if (live && col >= 0) {" : "if (col >= 0) {");
            o.ind++;
            o("T* p = &dy[(size_t)e * DSH + col];");
            if (add)
                o("*p += v;");
            else if (P.unit_weights)
                o("if (tile == 0 && !acc) *p = v; else *p += v;  // acc: add to an earlier call's dY");
            else
                o("if (tile == 0) *p = v; else *p += v;");
            o.ind--;
            o("}");
            o.ind--;
            o("}");
        }
    }
    o.ind--;
    o("}");
    if (radial) {
        // drho: sum over the slot's channel lanes; lane (r mod ct) of the slot writes (the first
        // group's first tile) or adds r
        o("if (drho) {");
        o.ind++;
        for (int r = 0; r < radial; ++r) o("dr", r, " = slot_sum<", g.ct, ">(dr", r, ");");
        for (int lo = 0; lo < radial; lo += g.ct) {
            o("{");
            o.ind++;
            o("T v = (T)0;");
            o("int col = -1;");
            for (int r = lo; r < std::min(radial, lo + g.ct); ++r) o("if (ul == ", r - lo, ") { v = dr", r, "; col = ", r, "; }");
            o("if (col >= 0) {");
            o.ind++;
            o("T* p = &drho[(size_t)e * NRAD + col];");
            o(gi == 0 ? "if (tile == 0) *p = v; else *p += v;" : "*p += v;");
            o.ind--;
            o("}");
            o.ind--;
            o("}");
        }
        o.ind--;
        o("}");
    }
    if (P.bwd_sched_barrier) o("__builtin_amdgcn_sched_barrier(0);");
    if (pf) {
        for (int r = 0; r < radial; ++r) o("rho", r, " = nrho", r, ";");
        for (int b : t.i2)
            for (int j = 0; j < n_of(P.sh[b].l); ++j) o("y", b, "_", j, " = ny", b, "_", j, ";");
        if (!P.unit_weights)
            for (int pi : g.paths) o("w", pi, " = nw", pi, ";");
        for (int q : t.slots)
            for (int k = 0; k < n_of(P.out[q].l); ++k) o("g", q, "_", k, " = ng", q, "_", k, ";");
        if (dbl) {
            for (int b : t.i2)
                for (int j = 0; j < n_of(P.sh[b].l); ++j) o("gy", b, "_", j, " = ngy", b, "_", j, ";");
            for (int pi : g.paths) o("gw", pi, " = ngw", pi, ";");
        }
    }
    if (rowmode) {
        o.ind--;
        o("}");
        o.ind--;
        o("}");
    } else {
    o("e = en;");
    o("n = nn;");
    o("en = enn;");
    o("nn = nnn;");
    o("tn = tnn;");
    o.ind--;
    o("}");  // edge loop
    o.ind--;
    o("}");  // t < t1
    }
    if (rowmode) {
        // each slot is its own row: no sum over slots or waves
        o("if (dx && live) {");
    } else {
    // sum the edge slots of the wave, then the waves of the workgroup (fixed order)
    for (int m = 32; m >= g.ct; m /= 2)
        for (int b : xb)
            for (int i = 0; i < n_of(P.ins[b].l); ++i) o(xadd("d" + std::to_string(b) + "_" + std::to_string(i), m));
    o("if (wpr > 1) {");
    o.ind++;
    o("if (wv > 0 && slot == 0) {");
    o.ind++;
    {
        int r = 0;
        for (int b : xb)
            for (int i = 0; i < n_of(P.ins[b].l); ++i, ++r)
                o("red[(wv - 1) * ", nx * g.ct, " + ", r * g.ct, " + ul] = d", b, "_", i, ";");
    }
    o.ind--;
    o("}");
    o("__syncthreads();");
    o("if (wv == 0) {");
    o.ind++;
    o("for (int v = 1; v < wpr; ++v) {");
    o.ind++;
    {
        int r = 0;
        for (int b : xb)
            for (int i = 0; i < n_of(P.ins[b].l); ++i, ++r)
                o("d", b, "_", i, " += red[(v - 1) * ", nx * g.ct, " + ", r * g.ct, " + ul];");
    }
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    o("__syncthreads();");
    o.ind--;
    o("}");
    o("if (dx && wv == 0 && slot == 0) {");
    }
    o.ind++;
    for (int b : xb) {
        const Irrep &ir = P.ins[b];
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.ins[bb].dim();
        if (!t.i1.count(b)) {
            // an input block no path reads: zero in every channel (its multiplicity may exceed the
            // channels this group's tiles cover), written once (not when adding to an earlier call)
            o(P.unit_weights ? "if (tile == 0 && !acc) {" : "if (tile == 0) {");
            o.ind++;
            o("for (int uu = ul; uu < ", ir.mul, "; uu += ", g.ct, ") {");
            o.ind++;
            for (int i = 0; i < n_of(ir.l); ++i) o("dx[(size_t)s * DX + ", off, " + uu * ", n_of(ir.l), " + ", i, "] = (T)0;");
            o.ind--;
            o("}");
            o.ind--;
            o("}");
            continue;
        }
        bool add = first_i1(b) >= 0 && first_i1(b) < gi;
        std::string guard = needs_mask(ir.mul, g) ? "if (u < " + std::to_string(ir.mul) + ") " : "";
        for (int i = 0; i < n_of(ir.l); ++i) {
            const std::string dst = "dx[(size_t)s * DX + " + std::to_string(off) + " + u * " + std::to_string(n_of(ir.l)) +
                                    " + " + std::to_string(i) + "]";
            if (add)
                o(guard, dst, " += d", b, "_", i, ";");
            else if (P.unit_weights)
                o(guard, "{ if (acc) ", dst, " += d", b, "_", i, "; else ", dst, " = d", b, "_", i, "; }");
            else
                o(guard, dst, " = d", b, "_", i, ";");
        }
    }
    o.ind--;
    o("}");
    if (radial) {
        o.ind--;
        o("}");  // senders of the chunk
        // dTheta partial of the chunk: sum the edge slots, then the waves (fixed order), then store
        std::vector<std::string> tas;
        for (int r = 0; r < radial; ++r)
            for (int pi : g.paths) tas.push_back("ta" + std::to_string(r) + "_" + std::to_string(pi));
        const int nt = (int)tas.size();
        for (int m = 32; m >= g.ct; m /= 2)
            for (auto &v : tas) o(xadd(v, m));
        o("if (wpr > 1) {");
        o.ind++;
        // in rounds of at most kRadialRound sums, so that the LDS buffer stays bounded
        for (int k0 = 0; k0 < nt; k0 += kRadialRound) {
            const int k1 = std::min(nt, k0 + kRadialRound), nk = k1 - k0;
            o("if (wv > 0 && slot == 0) {");
            o.ind++;
            for (int k = k0; k < k1; ++k) o("red[(wv - 1) * ", nk * g.ct, " + ", (k - k0) * g.ct, " + ul] = ", tas[k], ";");
            o.ind--;
            o("}");
            o("__syncthreads();");
            o("if (wv == 0) {");
            o.ind++;
            o("for (int v = 1; v < wpr; ++v) {");
            o.ind++;
            for (int k = k0; k < k1; ++k) o(tas[k], " += red[(v - 1) * ", nk * g.ct, " + ", (k - k0) * g.ct, " + ul];");
            o.ind--;
            o("}");
            o.ind--;
            o("}");
            o("__syncthreads();");
        }
        o.ind--;
        o("}");
        o("if (ws && wv == 0 && slot == 0) {");
        o.ind++;
        for (int r = 0; r < radial; ++r)
            for (int pi : g.paths) {
                const Path &p = P.paths[pi];
                const std::string guard = needs_mask(p.mul_in, g) ? "if (u < " + std::to_string(p.mul_in) + ") " : "";
                o(guard, "ws[(size_t)chunk * WN + ", (long)r * P.w_numel + p.w_off, " + u] = ta", r, "_", pi, ";");
            }
        o.ind--;
        o("}");
    }
    o.ind--;
    o("}");  // tile loop
    o.ind--;
    o("}");
    o("");
}

// LDS elements for the dx partials of waves 1..3 of a sender-pass workgroup: per group, the
// components of the input blocks it writes or adds (its own blocks; group 0 also the blocks no
// path touches) times its lanes per edge slot
int bwd_red_size(const std::vector<Group> &groups, const Plan &P)
{
    std::set<int> touched_any;
    for (const Group &g : groups)
        for (int pi : g.paths) touched_any.insert(P.paths[pi].i1);
    int m = 1;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
        const Group &g = groups[gi];
        std::set<int> blocks;
        for (int pi : g.paths) blocks.insert(P.paths[pi].i1);
        if (gi == 0)
            for (int b = 0; b < (int)P.ins.size(); ++b)
                if (!touched_any.count(b)) blocks.insert(b);
        int nx = 0;
        for (int b : blocks) nx += n_of(P.ins[b].l);
        m = std::max(m, 3 * nx * g.ct);
    }
    return m;
}

// Batched backward (use case A): rows-mode groups of the sender pass; one wave
// covers es rows, one launch per group (later groups add to dx / dY blocks an
// earlier group wrote), so every sum has a fixed order.
void emit_tpb_kernel(Out &o, const Plan &P)
{
    for (int gi = 0; gi < (int)P.bwd_groups.size(); ++gi) emit_bwd_group(o, P, gi, false, true);
    o("extern \"C\" __global__ void __launch_bounds__(256, ", P.bwd_waves_per_eu,
      ") cgtp_tp_bwd(const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ w, "
      "const T* __restrict__ g, T* __restrict__ dx, T* __restrict__ dy, T* __restrict__ dw, long nrows, long nblocks, "
      "int group)");
    o("{");
    o.ind++;
    o("const long blk = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("if (blk >= nblocks) return;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.bwd_groups.size(); ++gi)
        o("case ", gi, ": tpb_g", gi, "(blk, lane, x, y, w, g, dx, dy, dw, nrows); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// Sender-pass kernel: the backward (dbl = false) or the double backward's
// d/dx, d/dy, d/dW (dbl = true); slot_sum comes from the preamble.
void emit_bwd_kernel(Out &o, const Plan &P, bool dbl = false)
{
    const std::vector<Group> &groups = dbl ? P.dbl_groups : P.bwd_groups;
    for (int gi = 0; gi < (int)groups.size(); ++gi) emit_bwd_group(o, P, gi, dbl);
    o("// one workgroup of 64*wpr threads per sender; `group` selects the path group (launched in order)");
    o("extern \"C\" __global__ void __launch_bounds__(256, ", dbl ? P.dbl_bwd_waves_per_eu : P.bwd_waves_per_eu, ") ",
      dbl ? "cgtp_conv_dbwd_send" : P.unit_weights ? "cgtp_conv_uvw_bwd_xy" : "cgtp_conv_bwd",
      "(const int* __restrict__ t_row_ptr, "
      "const int* __restrict__ t_edge, const int* __restrict__ t_dst, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, const T* __restrict__ g, ",
      dbl ? "const T* __restrict__ ggx, const T* __restrict__ ggy, const T* __restrict__ ggw, " : "",
      "T* __restrict__ dx, T* __restrict__ dy, T* __restrict__ dw, long nnodes, int wpr, int group",
      P.unit_weights ? ", int acc" : "", ")");
    o("{");
    o.ind++;
    o("__shared__ T red[", bwd_red_size(groups, P), "];  // partial dx of waves 1..3");
    o("const long s = blockIdx.x;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("if (s >= nnodes) return;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)groups.size(); ++gi)
        o("case ", gi, ": ", dbl ? "dbs" : "bwd", "_g", gi, "(s, wv, lane, wpr, red, t_row_ptr, t_edge, t_dst, x, y, w, g, ",
          dbl ? "ggx, ggy, ggw, " : "", "dx, dy, dw", P.unit_weights ? ", acc" : "", "); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// ------------------------------------------------------------------------------------------
// Backward in receiver order (cgtp_conv_backward_receiver).  The edges of a contiguous range
// [e_lo, e_hi) of the receiver CSR are dealt to waves in blocks of `kper` consecutive edges, so
// the work per wave does not depend on the degree law.  A wave holds the output gradient g[n] of
// its current receiver in registers (reloaded when its edges cross into the next receiver) and
// gathers the sender row x[col[e]] per edge: the row it gathers is d_x wide, where the sender
// order gathers the d_out-wide gradient row.  Per edge and path, with B_ij = sum_k C_ijk g_k:
//   dW[e,p,u] = sum_i x_i sum_j B_ij y_j          (written once)
//   dY[e,j]  += W sum_i B_ij x_i, summed over the channel lanes (first writer stores, later add)
//   h[e,a_p + u(2l1+1) + i] += W sum_j B_ij y_j   (the edge's contribution to dx[col[e]])
// h goes to the caller's buffer (one row of d_x per edge of the range, only when dx is wanted);
// cgtp_conv_rbw_dx then sums, for every sender, the rows of its edges in the range (ascending
// edge id, from the transpose) into dx: the first range writes, later ranges add.  Every output
// element has one owner and a fixed summation order; no atomics.  One launch per forward path
// group (input blocks whole where they fit), in order; channel tiles are walked by the same wave.

void emit_find_receiver(Out &o)
{
    o("// largest n in [0, nrows) with row_ptr[n] <= e (row_ptr[0] = 0 <= e < row_ptr[nrows]):");
    o("// a 64-way search, all 64 lanes active, row_ptr non-decreasing so the probes that pass form a prefix");
    o("__device__ __forceinline__ long find_receiver(const int* __restrict__ row_ptr, long nrows, long e, int lane)");
    o("{");
    o.ind++;
    o("long lo = 0, hi = nrows;");
    o("while (hi - lo > 1) {");
    o.ind++;
    o("const long step = (hi - lo + 63) / 64;");
    o("const long p = lo + (long)lane * step;");
    o("const bool ok = p < hi && (long)row_ptr[p] <= e;");
    o("const unsigned long long m = __ballot(ok);");
    o("const long last = 63 - __clzll(m);");
    o("lo += last * step;");
    o("hi = (lo + step < hi) ? lo + step : hi;");
    o.ind--;
    o("}");
    o("return lo;");
    o.ind--;
    o("}");
    o("");
}

void emit_rbw_group(Out &o, const Plan &P, int gi)
{
    const std::vector<Group> &groups = P.rbw_groups;
    const Group &g = groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    Touch t = touched(P, g.paths);
    auto first_i1 = [&](int b) {
        for (int k = 0; k < (int)groups.size(); ++k)
            for (int pi : groups[k].paths)
                if (P.paths[pi].i1 == b) return k;
        return -1;
    };
    auto first_i2 = [&](int b) {
        for (int k = 0; k < (int)groups.size(); ++k)
            for (int pi : groups[k].paths)
                if (P.paths[pi].i2 == b) return k;
        return -1;
    };
    std::vector<int> xb, xz;  // input blocks whose h this group writes or adds; untouched blocks (zeroed)
    for (int b = 0; b < (int)P.ins.size(); ++b) {
        if (t.i1.count(b)) xb.push_back(b);
        if (gi == 0 && first_i1(b) < 0) xz.push_back(b);
    }
    std::vector<int> yb;  // SH blocks whose dY this group writes or adds
    for (int b = 0; b < (int)P.sh.size(); ++b)
        if (t.i2.count(b) || (gi == 0 && first_i2(b) < 0)) yb.push_back(b);
    auto xoff = [&](int b) {
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.ins[bb].dim();
        return off;
    };
    auto yoff = [&](int b) {
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.sh[bb].dim();
        return off;
    };
    auto ooff = [&](int q) {
        int off = 0;
        for (int qq = 0; qq < q; ++qq) off += P.out[qq].dim();
        return off;
    };

    o("__device__ __forceinline__ void rbw_g", gi,
      "(long blk, int lane, const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, const T* __restrict__ g, T* __restrict__ dy, "
      "T* __restrict__ dw, T* __restrict__ hb, long nrows, long e_lo, long e_hi, long kper)");
    o("{");
    o.ind++;
    o("const int slot = lane >> ", log2i(g.ct), ";");
    o("const int ul = lane & ", g.ct - 1, ";");
    o("const long eb0 = e_lo + blk * kper;");
    o("const long eb1 = (eb0 + kper < e_hi) ? eb0 + kper : e_hi;");
    o("const long n0 = find_receiver(row_ptr, nrows, eb0, lane);");
    o("for (int tile = 0; tile < ", g.tiles, "; ++tile) {");
    o.ind++;
    o("const int u = tile * ", g.ct, " + ul;");
    o("long e = eb0 + slot;");
    o("if (e < eb1) {");
    o.ind++;
    o("long n = n0;");
    o("long nend = row_ptr[n + 1];");
    o("while (nend <= e) { ++n; nend = row_ptr[n + 1]; }");
    auto load_g = [&](bool declare) {
        for (int q : t.slots) {
            const Irrep &ir = P.out[q];
            for (int k = 0; k < n_of(ir.l); ++k) {
                std::string ga = "g[(size_t)n * DOUT + " + std::to_string(ooff(q)) + " + u * " + std::to_string(n_of(ir.l)) +
                                 " + " + std::to_string(k) + "]";
                if (needs_mask(ir.mul, g))
                    o(declare ? "T " : "", "g", q, "_", k, " = (u < ", ir.mul, ") ? ", ga, " : (T)0;");
                else
                    o(declare ? "T " : "", "g", q, "_", k, " = ", ga, ";");
            }
        }
    };
    load_g(true);
    // operands of edge `ev` (sender `sv`) into registers <pre>x.., <pre>y.., <pre>w..
    auto load_ops = [&](const std::string &pre, const std::string &sv, const std::string &ev, bool declare) {
        const std::string Tq = declare ? "T " : "";
        for (int b : t.i1) {
            const Irrep &ir = P.ins[b];
            for (int i = 0; i < n_of(ir.l); ++i) {
                std::string addr = "x[(size_t)" + sv + " * DX + " + std::to_string(xoff(b)) + " + u * " +
                                   std::to_string(n_of(ir.l)) + " + " + std::to_string(i) + "]";
                if (needs_mask(ir.mul, g))
                    o(Tq, pre, "x", b, "_", i, " = (u < ", ir.mul, ") ? ", addr, " : (T)0;");
                else
                    o(Tq, pre, "x", b, "_", i, " = ", addr, ";");
            }
        }
        for (int b : t.i2)
            for (int j = 0; j < n_of(P.sh[b].l); ++j)
                o(Tq, pre, "y", b, "_", j, " = LD_STREAM(&y[(size_t)", ev, " * DSH + ", yoff(b) + j, "]);");
        for (int pi : g.paths) {
            const Path &p = P.paths[pi];
            std::string wa = "LD_STREAM(&w[(size_t)" + ev + " * WROW + " + std::to_string(p.w_off) + " + u])";
            if (needs_mask(p.mul_in, g))
                o(Tq, pre, "w", pi, " = (u < ", p.mul_in, ") ? ", wa, " : (T)0;");
            else
                o(Tq, pre, "w", pi, " = ", wa, ";");
        }
    };
    const bool pf = P.rbw_prefetch;
    if (pf) {
        // pipeline: sender ids two edges ahead, operands one ahead (indices clamped to the block)
        o("long en = (e + ", g.es, " < eb1) ? e + ", g.es, " : e;");
        o("long s = col[e], sn = col[en];");
        load_ops("", "s", "e", true);
    }
    o("for (; e < eb1; e += ", g.es, ") {");
    o.ind++;
    if (pf) {
        o("const long enn = (en + ", g.es, " < eb1) ? en + ", g.es, " : en;");
        o("const long snn = col[enn];");
        load_ops("n", "sn", "en", true);
    }
    o("if (e >= nend) {");
    o.ind++;
    o("do { ++n; nend = row_ptr[n + 1]; } while (nend <= e);");
    load_g(false);
    o.ind--;
    o("}");
    if (!pf) {
        o("const long s = col[e];");
        load_ops("", "s", "e", true);
    }
    for (int b : xb)
        for (int i = 0; i < n_of(P.ins[b].l); ++i) o("T d", b, "_", i, " = (T)0;");
    for (int b : yb)
        for (int j = 0; j < n_of(P.sh[b].l); ++j) o("T h", b, "_", j, " = (T)0;");
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        std::map<std::pair<int, int>, std::vector<const Nonzero *>> byij;
        for (const Nonzero &z : p.nz) byij[{z.i, z.j}].push_back(&z);
        o("{");
        o.ind++;
        for (auto &kv : byij)
            o("const T B", kv.first.first, "_", kv.first.second, " = ",
              cg_sum_k(kv.second, "g" + std::to_string(p.slot) + "_", f64), ";");
        std::map<int, std::vector<int>> rows, cols;
        for (auto &kv : byij) {
            rows[kv.first.first].push_back(kv.first.second);
            cols[kv.first.second].push_back(kv.first.first);
        }
        // fx_i = sum_j B_ij y_j ; fy_j = sum_i B_ij x_i
        for (auto &kv : rows) {
            std::ostringstream e;
            e << "B" << kv.first << "_" << kv.second[0] << " * y" << p.i2 << "_" << kv.second[0];
            for (size_t m = 1; m < kv.second.size(); ++m) {
                std::ostringstream f;
                f << "FMA(B" << kv.first << "_" << kv.second[m] << ", y" << p.i2 << "_" << kv.second[m] << ", " << e.str()
                  << ")";
                e.str(f.str());
            }
            o("const T fx", kv.first, " = ", e.str(), ";");
        }
        for (auto &kv : cols) {
            std::ostringstream e;
            e << "B" << kv.second[0] << "_" << kv.first << " * x" << p.i1 << "_" << kv.second[0];
            for (size_t m = 1; m < kv.second.size(); ++m) {
                std::ostringstream f;
                f << "FMA(B" << kv.second[m] << "_" << kv.first << ", x" << p.i1 << "_" << kv.second[m] << ", " << e.str()
                  << ")";
                e.str(f.str());
            }
            o("const T fy", kv.first, " = ", e.str(), ";");
        }
        {
            // dW = sum_i x_i fx_i
            std::ostringstream e;
            bool first = true;
            for (auto &kv : rows) {
                if (first) {
                    e << "x" << p.i1 << "_" << kv.first << " * fx" << kv.first;
                    first = false;
                } else {
                    std::ostringstream f;
                    f << "FMA(x" << p.i1 << "_" << kv.first << ", fx" << kv.first << ", " << e.str() << ")";
                    e.str(f.str());
                }
            }
            std::string guard = needs_mask(p.mul_in, g) ? "(u < " + std::to_string(p.mul_in) + ") && " : "";
            o("if (", guard, "dw) ST_STREAM(", e.str(), ", &dw[(size_t)e * WROW + ", p.w_off, " + u]);");
        }
        for (auto &kv : rows)
            o("d", p.i1, "_", kv.first, " = FMA(w", pi, ", fx", kv.first, ", d", p.i1, "_", kv.first, ");");
        for (auto &kv : cols)
            o("h", p.i2, "_", kv.first, " = FMA(w", pi, ", fy", kv.first, ", h", p.i2, "_", kv.first, ");");
        o.ind--;
        o("}");
        // one path at a time: interleaving the paths' temporaries would multiply the live registers
        if (P.rbw_sched_barrier) o("__builtin_amdgcn_sched_barrier(0);");
    }
    // the edge's contribution to dx of its sender: row (e - e_lo) of hb
    o("if (hb) {");
    o.ind++;
    o("T* hr = hb + (size_t)(e - e_lo) * DX;");
    if (!xz.empty()) {
        // input blocks no path reads: their dx is zero (all channels, once)
        o("if (tile == 0) {");
        o.ind++;
        for (int b : xz) {
            o("for (int uu = ul; uu < ", P.ins[b].mul, "; uu += ", g.ct, ") {");
            o.ind++;
            for (int i = 0; i < n_of(P.ins[b].l); ++i) o("hr[", xoff(b), " + uu * ", n_of(P.ins[b].l), " + ", i, "] = (T)0;");
            o.ind--;
            o("}");
        }
        o.ind--;
        o("}");
    }
    for (int b : xb) {
        const Irrep &ir = P.ins[b];
        const bool add = first_i1(b) >= 0 && first_i1(b) < gi;
        std::string guard = needs_mask(ir.mul, g) ? "if (u < " + std::to_string(ir.mul) + ") " : "";
        for (int i = 0; i < n_of(ir.l); ++i)
            o(guard, "hr[", xoff(b), " + u * ", n_of(ir.l), " + ", i, "] ", add ? "+=" : "=", " d", b, "_", i, ";");
    }
    o.ind--;
    o("}");
    // dY: sum over the slot's channel lanes; lane (j mod ct) of the slot writes or adds column j
    o("if (dy) {");
    o.ind++;
    std::vector<std::pair<int, std::string>> hs;
    for (int b : yb)
        for (int jj = 0; jj < n_of(P.sh[b].l); ++jj)
            hs.push_back({yoff(b) + jj, "h" + std::to_string(b) + "_" + std::to_string(jj)});
    for (auto &h : hs) o(h.second, " = slot_sum<", g.ct, ">(", h.second, ");");
    for (size_t r = 0; r * g.ct < hs.size(); ++r) {
        const size_t lo = r * g.ct, hi = std::min(hs.size(), (r + 1) * g.ct);
        for (int add = 0; add < 2; ++add) {
            std::vector<std::pair<size_t, int>> sel;
            for (size_t c = lo; c < hi; ++c) {
                int colj = hs[c].first, blk = 0, acc = 0;
                for (int b = 0; b < (int)P.sh.size(); ++b) {
                    if (colj < acc + P.sh[b].dim()) {
                        blk = b;
                        break;
                    }
                    acc += P.sh[b].dim();
                }
                bool is_add = first_i2(blk) >= 0 && first_i2(blk) < gi;
                if ((int)is_add == add) sel.push_back({c - lo, colj});
            }
            if (sel.empty()) continue;
            o("{");
            o.ind++;
            o("T v = (T)0;");
            o("int cj = -1;");
            for (auto &sc : sel) o("if (ul == ", sc.first, ") { v = ", hs[lo + sc.first].second, "; cj = ", sc.second, "; }");
            o("if (cj >= 0) {");
            o.ind++;
            o("T* p = &dy[(size_t)e * DSH + cj];");
            if (add)
                o("*p += v;");
            else
                o("if (tile == 0) *p = v; else *p += v;");
            o.ind--;
            o("}");
            o.ind--;
            o("}");
        }
    }
    o.ind--;
    o("}");
    if (pf) {
        for (int b : t.i1)
            for (int i = 0; i < n_of(P.ins[b].l); ++i) o("x", b, "_", i, " = nx", b, "_", i, ";");
        for (int b : t.i2)
            for (int j = 0; j < n_of(P.sh[b].l); ++j) o("y", b, "_", j, " = ny", b, "_", j, ";");
        for (int pi : g.paths) o("w", pi, " = nw", pi, ";");
        o("en = enn;");
        o("sn = snn;");
    }
    o.ind--;
    o("}");  // edge loop
    o.ind--;
    o("}");  // e < eb1
    o.ind--;
    o("}");  // tile loop
    o.ind--;
    o("}");
    o("");
}

void emit_rbw_kernels(Out &o, const Plan &P)
{
    emit_find_receiver(o);
    for (int gi = 0; gi < (int)P.rbw_groups.size(); ++gi) emit_rbw_group(o, P, gi);
    o("// one wave per block of kper consecutive edges of [e_lo, e_hi); `group` selects the path group (in order)");
    o("extern \"C\" __global__ void __launch_bounds__(256, ", P.rbw_waves_per_eu,
      ") cgtp_conv_rbw(const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, const T* __restrict__ g, T* __restrict__ dy, "
      "T* __restrict__ dw, T* __restrict__ hb, long nrows, long e_lo, long e_hi, long kper, int group)");
    o("{");
    o.ind++;
    o("const long blk = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("if (e_lo + blk * kper >= e_hi) return;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.rbw_groups.size(); ++gi)
        o("case ", gi, ": rbw_g", gi, "(blk, lane, row_ptr, col, x, y, w, g, dy, dw, hb, nrows, e_lo, e_hi, kper); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
    // dx of every sender from the rows of its edges in [e_lo, e_hi): one wave per sender, lanes over
    // columns; edge ids ascend inside a sender's part of the transpose, so the range is found with
    // two counts over that part
    const int nc = (P.d_x + 63) / 64;
    o("// dx[s] (first range: =, later ranges: +=) sum of hb rows of the sender's edges in [e_lo, e_hi),");
    o("// in ascending edge id; one wave per sender, lane c holds columns c, c + 64, ...");
    o("extern \"C\" __global__ void __launch_bounds__(256) cgtp_conv_rbw_dx(const int* __restrict__ t_row_ptr, "
      "const int* __restrict__ t_edge, const T* __restrict__ hb, T* __restrict__ dx, long nnodes, long e_lo, "
      "long e_hi, int first)");
    o("{");
    o.ind++;
    o("const long s = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("if (s >= nnodes) return;");
    o("const int t0 = t_row_ptr[s], t1 = t_row_ptr[s + 1];");
    o("int ta = t0, tb = t0;");
    o("for (int base = t0; base < t1; base += 64) {");
    o.ind++;
    o("const int tt = base + lane;");
    o("const long ev = tt < t1 ? (long)t_edge[tt] : e_hi;");
    o("ta += __popcll(__ballot(tt < t1 && ev < e_lo));");
    o("tb += __popcll(__ballot(tt < t1 && ev < e_hi));");
    o.ind--;
    o("}");
    o("if (!first && ta == tb) return;");
    for (int m = 0; m < nc; ++m) o("T a", m, " = (T)0;");
    // edge ids of 64 rows at a time, one per lane, then broadcast: the row loads of consecutive
    // edges do not wait for a scalar index load each, and two rows are in flight per step
    o("for (int base = ta; base < tb; base += 64) {");
    o.ind++;
    o("const int cnt = (tb - base < 64) ? tb - base : 64;");
    o("const int ev = (lane < cnt) ? t_edge[base + lane] : 0;");
    auto row_loads = [&](const std::string &r, const std::string &v) {
        for (int m = 0; m < nc; ++m) {
            if ((m + 1) * 64 <= P.d_x)
                o("const T ", v, m, " = LD_STREAM(&", r, "[", m * 64, "]);");
            else
                o("const T ", v, m, " = (lane + ", m * 64, " < DX) ? LD_STREAM(&", r, "[", m * 64, "]) : (T)0;");
        }
    };
    o("int j = 0;");
    o("for (; j + 1 < cnt; j += 2) {");
    o.ind++;
    o("const T* r0 = hb + (size_t)(__builtin_amdgcn_readlane(ev, j) - e_lo) * DX + lane;");
    o("const T* r1 = hb + (size_t)(__builtin_amdgcn_readlane(ev, j + 1) - e_lo) * DX + lane;");
    row_loads("r0", "p");
    row_loads("r1", "q");
    for (int m = 0; m < nc; ++m) o("a", m, " += p", m, ";");
    for (int m = 0; m < nc; ++m) o("a", m, " += q", m, ";");
    o.ind--;
    o("}");
    o("if (j < cnt) {");
    o.ind++;
    o("const T* r0 = hb + (size_t)(__builtin_amdgcn_readlane(ev, j) - e_lo) * DX + lane;");
    row_loads("r0", "p");
    for (int m = 0; m < nc; ++m) o("a", m, " += p", m, ";");
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    o("T* d = dx + (size_t)s * DX + lane;");
    for (int m = 0; m < nc; ++m) {
        std::string guard = (m + 1) * 64 <= P.d_x ? "" : "if (lane + " + std::to_string(m * 64) + " < DX) ";
        o(guard, "d[", m * 64, "] = first ? a", m, " : d[", m * 64, "] + a", m, ";");
    }
    o.ind--;
    o("}");
    o("");
}

// ------------------------------------------------------------------------------------------
// uvw batched product: sparse CG contraction on VALU, dense multiplicity mixing
// on MFMA (16x16x4).  One wave covers 16 rows; lane l works on row l % 16 and on
// input channels u = 4c + l / 16 for the four channel chunks c.  The contraction
// with y depends only on the row, so for each path and output component k the
// column A[i] = sum_j C_ijk y_j is formed once (literal constants) and reused for
// the four chunks: t_c = sum_i A[i] x[row, 4c + l/16, i] (LunaTP page, Abstract:
// multi-level reuse).  t_c is directly the MFMA B operand and W_p[u][w = l % 16]
// the A operand, so
//   D_{q,k}[w][row] += sum_u W_p[u][w] t_p[row, u, k]
// accumulates the output block q = slot(p) in registers across paths and
// chunks.  Lane l ends holding out[row = l % 16][w][k] in register v, with
// w = 4 (l / 16) + v (fp32 instruction) or w = l / 16 + 4 v (fp64 instruction).
void emit_uvw_group(Out &o, const Plan &P, int gi)
{
    const Group &g = P.uvw_groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    Touch t = touched(P, g.paths);
    int chunks = 0;
    for (int pi : g.paths) chunks = std::max(chunks, (P.paths[pi].mul_in + 3) / 4);
    // output multiplicities above 16 take one wave per 16-wide tile of output channels (wt);
    // plans within one tile generate no tile index at all
    const bool tiled = uvw_out_tiles(P) > 1;
    o("__device__ __forceinline__ void uvw_g", gi,
      "(long blk, int lane, const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ w, "
      "T* __restrict__ out, long nrows", tiled ? ", int wt" : "", ")");
    o("{");
    o.ind++;
    if (tiled) o("const int wcol = wt * 16 + (lane & 15);  // output channel of this lane's A operand");
    o("const long row = blk * 16 + (lane & 15);");
    o("const int usub = lane >> 4;");
    o("const bool live = row < nrows;");
    o("const long rr = live ? row : nrows - 1;  // rows past the end read row nrows-1 and are never stored");
    for (int q : t.slots)
        for (int k = 0; k < n_of(P.out[q].l); ++k) o("V4 a", q, "_", k, " = {0, 0, 0, 0};");
    for (int b : t.i2) {
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.sh[bb].dim();
        for (int j = 0; j < n_of(P.sh[b].l); ++j) o("const T y", b, "_", j, " = y[(size_t)rr * DSH + ", off + j, "];");
    }
    // paths grouped by input block: that block's x is loaded for all chunks once
    std::map<int, std::vector<int>> by_i1;
    for (int pi : g.paths) by_i1[P.paths[pi].i1].push_back(pi);
    // A operands W_p[u][w] (u = 4c + lane/16, w = lane % 16) run one path ahead in two register
    // sets: path t's are loaded when path t - 1 starts (unconditionally, from a clamped element;
    // the mask is applied where they are used), so that their latency is covered by a path's work
    std::vector<int> order;
    for (auto &kv : by_i1)
        for (int pi : kv.second) order.push_back(pi);
    const std::string wc = tiled ? "wcol" : "(lane & 15)";
    auto wmask_of = [&](const Path &p, int c) { return 4 * c + 3 >= p.mul_in || p.mul_out < 16 || tiled; };
    auto load_w = [&](int t) {
        const Path &p = P.paths[order[t]];
        for (int c = 0; c < chunks; ++c) {
            const std::string u = "(" + std::to_string(4 * c) + " + usub)";
            if (wmask_of(p, c))
                o("wv", t % 2, "_", c, " = w[", p.w_off, " + (", u, " < ", p.mul_in, " ? ", u, " : 0) * ", p.mul_out, " + (", wc,
                  " < ", p.mul_out, " ? ", wc, " : 0)];");
            else
                o("wv", t % 2, "_", c, " = w[", p.w_off, " + ", u, " * ", p.mul_out, " + (lane & 15)];");
        }
    };
    for (int set = 0; set < 2; ++set)
        for (int c = 0; c < chunks; ++c) o("T wv", set, "_", c, " = (T)0;");
    if (!order.empty()) load_w(0);
    int tpath = 0;
    for (auto &kv : by_i1) {
        const int b = kv.first;
        const Irrep &ir = P.ins[b];
        int off = 0;
        for (int bb = 0; bb < b; ++bb) off += P.ins[bb].dim();
        o("{");
        o.ind++;
        for (int c = 0; c < chunks; ++c) {
            const bool mask = 4 * c + 3 >= ir.mul;
            std::string u = "(" + std::to_string(4 * c) + " + usub)";
            for (int i = 0; i < n_of(ir.l); ++i) {
                std::string addr = "(size_t)rr * DX + " + std::to_string(off) + " + " + (mask ? "(" + u + " < " +
                                   std::to_string(ir.mul) + " ? " + u + " : 0)" : u) + " * " + std::to_string(n_of(ir.l)) +
                                   " + " + std::to_string(i);
                if (mask)
                    o("const T x", c, "_", i, " = ", u, " < ", ir.mul, " ? x[", addr, "] : (T)0;");
                else
                    o("const T x", c, "_", i, " = x[", addr, "];");
            }
        }
        for (int pi : kv.second) {
            const Path &p = P.paths[pi];
            const int tp = tpath++;
            o("{");
            o.ind++;
            // this path's A operands (zero outside the block), then the next path's loads
            for (int c = 0; c < chunks; ++c) {
                const std::string u = "(" + std::to_string(4 * c) + " + usub)";
                if (wmask_of(p, c))
                    o("const T wa", c, " = (", u, " < ", p.mul_in, " && ", wc, " < ", p.mul_out, ") ? wv", tp % 2, "_", c, " : (T)0;");
                else
                    o("const T wa", c, " = wv", tp % 2, "_", c, ";");
            }
            if (tp + 1 < (int)order.size()) {
                load_w(tp + 1);
                o("__builtin_amdgcn_sched_barrier(0);");
            }
            std::map<int, std::map<int, std::vector<const Nonzero *>>> byki;  // k -> i -> nonzeros
            for (const Nonzero &z : p.nz) byki[z.k][z.i].push_back(&z);
            for (auto &kk : byki) {
                const int k = kk.first;
                o("{");
                o.ind++;
                for (auto &ii : kk.second) {
                    const auto &v = ii.second;
                    std::ostringstream e;
                    e << lit(v[0]->c, f64) << " * y" << p.i2 << "_" << v[0]->j;
                    for (size_t n = 1; n < v.size(); ++n) {
                        std::ostringstream f;
                        f << "FMA(" << lit(v[n]->c, f64) << ", y" << p.i2 << "_" << v[n]->j << ", " << e.str() << ")";
                        e.str(f.str());
                    }
                    o("const T A", ii.first, " = ", e.str(), ";");
                }
                for (int c = 0; c < chunks; ++c) {
                    std::ostringstream e;
                    bool first = true;
                    for (auto &ii : kk.second) {
                        if (first) {
                            e << "A" << ii.first << " * x" << c << "_" << ii.first;
                            first = false;
                        } else {
                            std::ostringstream f;
                            f << "FMA(A" << ii.first << ", x" << c << "_" << ii.first << ", " << e.str() << ")";
                            e.str(f.str());
                        }
                    }
                    o("a", p.slot, "_", k, " = MFMA(wa", c, ", ", e.str(), ", a", p.slot, "_", k, ");");
                }
                o.ind--;
                o("}");
            }
            o.ind--;
            o("}");
        }
        o.ind--;
        o("}");
    }
    o("if (live) {");
    o.ind++;
    o("T* orow = out + (size_t)row * DOUT;");
    for (int q : t.slots) {
        const Irrep &ir = P.out[q];
        int off = 0;
        for (int qq = 0; qq < q; ++qq) off += P.out[qq].dim();
        for (int v = 0; v < 4; ++v) {
            o("{");
            o.ind++;
            // D row held in register v of this lane: 4 (lane / 16) + v for the fp32
            // instruction, lane / 16 + 4 v for the fp64 one
            const std::string tile0 = tiled ? "wt * 16 + " : "";
            if (f64)
                o("const int wo = ", tile0, "usub + ", 4 * v, ";");
            else
                o("const int wo = ", tile0, "4 * usub + ", v, ";");
            const bool guard = ir.mul < 16 || tiled;
            if (guard) o("if (wo < ", ir.mul, ") {");
            for (int k = 0; k < n_of(ir.l); ++k)
                o("orow[", off, " + wo * ", n_of(ir.l), " + ", k, "] = a", q, "_", k, "[", v, "];");
            if (guard) o("}");
            o.ind--;
            o("}");
        }
    }
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    o("");
}

void emit_mfma_defs(Out &o, const Plan &P)
{
    const bool f64 = P.dtype == CGTP_F64;
    o("typedef ", f64 ? "double" : "float", " V4 __attribute__((ext_vector_type(4)));");
    if (f64)
        o("#define MFMA(a, b, c) __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0)");
    else
        o("#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0)");
}

void emit_uvw_kernel(Out &o, const Plan &P)
{
    for (int gi = 0; gi < (int)P.uvw_groups.size(); ++gi) emit_uvw_group(o, P, gi);
    o("// one wave per (group, 16-row block), group-major so that the waves resident at any time");
    o("// mostly run the same group's code");
    o("extern \"C\" __global__ void __launch_bounds__(256, ", P.uvw_waves_per_eu,
      ") cgtp_tp_uvw(const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ w, "
      "T* __restrict__ out, long nrows, long nblocks)");
    o("{");
    o.ind++;
    o("const long wave = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    const int tiles = uvw_out_tiles(P);
    if (tiles > 1) {
        // waves are (group, output tile, block), block fastest
        o("const long per_group = nblocks * ", tiles, ";");
        o("const int group = (int)(wave / per_group);");
        o("const long rest = wave - (long)group * per_group;");
        o("const int wt = (int)(rest / nblocks);");
        o("const long blk = rest - (long)wt * nblocks;");
    } else {
        o("const int group = (int)(wave / nblocks);");
        o("const long blk = wave - (long)group * nblocks;");
    }
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.uvw_groups.size(); ++gi)
        o("case ", gi, ": uvw_g", gi, "(blk, lane, x, y, w, out, nrows", tiles > 1 ? ", wt" : "", "); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// ------------------------------------------------------------------------------------------
// uvw convolution (shared weights): one workgroup per tile of 16 receivers
// (16 / rpw waves, rpw receivers each) and one launch per path group.  Edge stream: lanes are input
// channels (edge slots when there are fewer than 64), and per receiver the
// unweighted sums T_p[u][k] = sum over its edges of sum_ij C_ijk x[s,u,i] y[e,j]
// stay in registers (Sobek page, Abstract: edge-local products consumed into
// bounded receiver-side state).  T is staged in LDS as [p,k][u][row], the 16 rows of each u
// XOR-swizzled (see emit_tsw).  Mixing:
// out[n, q, w, k] (+)= sum_p sum_u W_p[u][w] T_p[n][u][k] on MFMA 16x16x4 with
// the 16 receivers as the B columns (A = W_p[u][w = lane % 16], B = T[row =
// lane % 16][u = 4c + lane / 16][k]).  A slot's first group writes it, later
// groups (later launches) add, so every sum has a fixed order.
int uvc_mu_pad(const Path &p) { return (p.mul_in + 3) / 4 * 4; }

// Position of T[u][row] inside a [u][row] block: the row index XOR ((u ^ (u >> 4)) & 15), so that
// the three access patterns (the edge stream writing 64 consecutive u of one row, the forward's
// MFMA reading 4 u x 16 rows, the dW pass reading 16 u x 4 rows) each touch distinct banks
// (fp32; two words per fp64 element, the fewest possible).  Plain [u][row] strides the latter
// two by 16 words.
void emit_tsw(Out &o)
{
    o("#ifndef TSW");
    o("#define TSW(u, r) ((u) * 16 + ((r) ^ (((u) ^ ((u) >> 4)) & 15)))");
    o("#endif");
}

// uvw convolution, edge stream of one path group: each wave accumulates the unweighted per-path
// sums T_p[u][k] of its receivers' edges (rows r of the tile `tile`) and stages them in LDS as
// [p,k][u][row] at the offsets `loff`.  Shared by the forward and the dW pass.
void emit_uvc_phase_a(Out &o, const Plan &P, const Group &g, std::map<int, int> &loff, bool rad = false)
{
    Touch t = touched(P, g.paths);
    const bool f64 = P.dtype == CGTP_F64;
    o("const int slot = lane >> ", log2i(g.ct), ";");
    o("const int ul = lane & ", g.ct - 1, ";");
    const int nw = 16 / P.uvc_rpw;  // waves per workgroup
    o("for (int m = 0; m < ", P.uvc_rpw, "; ++m) {");
    o.ind++;
    o("const int r = wv + ", nw, " * m;  // receiver of the tile handled by this wave");
    o("const long idx = tile * 16 + r;");
    o("const bool live = idx < nrows;");
    o("const long n = live ? (order ? (long)order[idx] : idx) : 0;");
    o("for (int ctile = 0; ctile < ", g.tiles, "; ++ctile) {");
    o.ind++;
    o("const int u = ctile * ", g.ct, " + ul;");
    for (int pi : g.paths)
        for (int k = 0; k < n_of(P.paths[pi].l3); ++k) o("T t", pi, "_", k, " = (T)0;");
    o("const int e0 = live ? row_ptr[n] : 0, e1 = live ? row_ptr[n + 1] : 0;");
    o("if (e0 < e1) {");
    o.ind++;
    // operands: x of the sender (gathered), y of the edge; senders two ahead, operands one ahead
    auto loads = [&](const std::string &pre, const std::string &si, const std::string &ei, bool declare) {
        const std::string Ty = declare ? "T " : "";
        for (int b : t.i1) {
            const Irrep &ir = P.ins[b];
            int off = 0;
            for (int pi : g.paths)
                if (P.paths[pi].i1 == b) off = P.paths[pi].a;
            const bool m = needs_mask(ir.mul, g);
            for (int i = 0; i < n_of(ir.l); ++i) {
                std::ostringstream addr;
                addr << "x[(size_t)" << si << " * DX + " << off << " + " << (m ? "(u < " + std::to_string(ir.mul) + " ? u : 0)" : "u")
                     << " * " << n_of(ir.l) << " + " << i << "]";
                if (m)
                    o(Ty, pre, "x", b, "_", i, " = (u < ", ir.mul, ") ? ", addr.str(), " : (T)0;");
                else
                    o(Ty, pre, "x", b, "_", i, " = ", addr.str(), ";");
            }
        }
        // radial variant: the edge's SH values scaled by its radial feature rr (rho_e[rr] y_e)
        if (rad) o("const T ", pre, "rs = rho[(size_t)", ei, " * nrad + rr];");
        for (int b : t.i2) {
            int off = 0;
            for (int pi : g.paths)
                if (P.paths[pi].i2 == b) off = P.paths[pi].b;
            for (int j = 0; j < n_of(P.sh[b].l); ++j)
                o(Ty, pre, "y", b, "_", j, " = y[(size_t)", ei, " * DSH + ", off + j, "]", rad ? " * " + pre + "rs" : "", ";");
        }
    };
    auto copy = [&]() {
        for (int b : t.i1)
            for (int i = 0; i < n_of(P.ins[b].l); ++i) o("cx", b, "_", i, " = nx", b, "_", i, ";");
        for (int b : t.i2)
            for (int j = 0; j < n_of(P.sh[b].l); ++j) o("cy", b, "_", j, " = ny", b, "_", j, ";");
    };
    o("int e = e0 + slot;");
    o("int ec = e < e1 ? e : e1 - 1;");
    o("int s = col[ec];");
    o("int en = (e + ", g.es, " < e1) ? e + ", g.es, " : e1 - 1;");
    o("int sn = col[en];");
    loads("c", "s", "ec", true);
    o("for (; e < e1; e += ", g.es, ") {");
    o.ind++;
    o("const int enn = (e + ", 2 * g.es, " < e1) ? e + ", 2 * g.es, " : e1 - 1;");
    o("const int snn = col[enn];");
    loads("n", "sn", "en", true);
    // keep the next edge's loads ahead of this edge's arithmetic (left alone, the scheduler sinks
    // them to the end of the iteration and every edge waits for its own operands)
    if (P.uvc_sched_barrier) o("__builtin_amdgcn_sched_barrier(0);");
    for (auto &pr : pairs_of(P, g.paths)) {
        int i1 = pr.first.first, i2 = pr.first.second;
        std::set<std::pair<int, int>> used;
        for (int pi : pr.second)
            for (const Nonzero &z : P.paths[pi].nz) used.insert({z.i, z.j});
        o("{");
        o.ind++;
        for (auto &ij : used)
            o("const T q", ij.first, "_", ij.second, " = cx", i1, "_", ij.first, " * cy", i2, "_", ij.second, ";");
        for (int pi : pr.second) {
            std::map<int, std::vector<const Nonzero *>> byk;
            for (const Nonzero &z : P.paths[pi].nz) byk[z.k].push_back(&z);
            // the running sum is the innermost addend of the chain: one FMA per nonzero and no
            // separate add per (path, k) block
            for (auto &kv : byk) {
                std::string e = "t" + std::to_string(pi) + "_" + std::to_string(kv.first);
                for (const Nonzero *z : kv.second)
                    e = "FMA(" + lit(z->c, f64) + ", q" + std::to_string(z->i) + "_" + std::to_string(z->j) + ", " + e + ")";
                o("t", pi, "_", kv.first, " = ", e, ";");
            }
        }
        o.ind--;
        o("}");
    }
    copy();
    o("en = enn;");
    o("sn = snn;");
    o.ind--;
    o("}");  // edge loop
    o.ind--;
    o("}");  // e0 < e1
    for (int m = 32; m >= g.ct; m /= 2)
        for (int pi : g.paths)
            for (int k = 0; k < n_of(P.paths[pi].l3); ++k) o(xadd("t" + std::to_string(pi) + "_" + std::to_string(k), m));
    o("if (slot == 0) {");
    o.ind++;
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        const int mp = uvc_mu_pad(p);
        for (int k = 0; k < n_of(p.l3); ++k)
            o("if (u < ", mp, ") lds[", loff[pi] + 16 * mp * k, " + TSW(u, r)] = t", pi, "_", k, ";");
    }
    o.ind--;
    o("}");
    o.ind--;
    o("}");  // channel tiles
    o.ind--;
    o("}");  // receivers of the wave
}

void emit_uvc_group(Out &o, const Plan &P, int gi, int variant = 0)
{
    const bool acc_variant = variant > 0, rad = variant == 2;
    const Group &g = P.uvc_groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    Touch t = touched(P, g.paths);
    auto first_group_of_slot = [&](int q) {
        for (int k = 0; k < (int)P.uvc_groups.size(); ++k)
            for (int pi : P.uvc_groups[k].paths)
                if (P.paths[pi].slot == q) return k;
        return -1;
    };
    // LDS offset (in elements) of each path's T block
    std::map<int, int> loff;
    int lds_elems = 0;
    for (int pi : g.paths) {
        loff[pi] = lds_elems;
        lds_elems += 16 * uvc_mu_pad(P.paths[pi]) * n_of(P.paths[pi].l3);
    }
    emit_tsw(o);
    o("__device__ __forceinline__ void ", rad ? "uvcr_g" : acc_variant ? "uvca_g" : "uvc_g", gi,
      "(long tile, int wv, int lane, const int* __restrict__ row_ptr, const int* __restrict__ col, "
      "const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ w, T* __restrict__ out, long nrows, "
      "const int* __restrict__ order, T* lds", acc_variant ? ", int acc" : "",
      rad ? ", const T* __restrict__ rho, int nrad, int rr" : "", ")");
    o("{");
    o.ind++;
    const int nw = 16 / P.uvc_rpw;  // waves per workgroup
    emit_uvc_phase_a(o, P, g, loff, rad);
    o("__syncthreads();");
    // mixing on MFMA: items (slot q, 16-wide block of output channels), round-robin over the waves
    o("const int usub = lane >> 4;");
    o("const int row = lane & 15;");
    o("const long oidx = tile * 16 + row;");
    o("const bool olive = oidx < nrows;");
    o("const long on = olive ? (order ? (long)order[oidx] : oidx) : 0;");
    o("T* orow = out + (size_t)on * DOUT;");
    int item = 0;
    for (int q : t.slots) {
        const Irrep &ir = P.out[q];
        int ooff = 0;
        for (int qq = 0; qq < q; ++qq) ooff += P.out[qq].dim();
        const bool add = first_group_of_slot(q) < gi;
        const int wtiles = (ir.mul + 15) / 16;
        for (int wt = 0; wt < wtiles; ++wt, ++item) {
            o("if (wv == ", item % nw, ") {");
            o.ind++;
            for (int k = 0; k < n_of(ir.l); ++k) o("V4 d", k, " = {0, 0, 0, 0};");
            for (int pi : g.paths) {
                const Path &p = P.paths[pi];
                if (p.slot != q) continue;
                const int mp = uvc_mu_pad(p);
                o("{");
                o.ind++;
                for (int c = 0; c < mp / 4; ++c) {
                    std::string u = "(" + std::to_string(4 * c) + " + usub)";
                    std::string wcol = "(" + std::to_string(16 * wt) + " + row)";
                    const bool wmask = 4 * c + 3 >= p.mul_in || 16 * wt + 15 >= p.mul_out;
                    if (wmask) {
                        o("const bool wok", c, " = ", u, " < ", p.mul_in, " && ", wcol, " < ", p.mul_out, ";");
                        o("const T wv", c, " = w[", p.w_off, " + (wok", c, " ? ", u, " * ", p.mul_out, " + ", wcol, " : 0)];");
                        o("const T wa", c, " = wok", c, " ? wv", c, " : (T)0;");
                    } else {
                        o("const T wa", c, " = w[", p.w_off, " + ", u, " * ", p.mul_out, " + ", wcol, "];");
                    }
                }
                for (int k = 0; k < n_of(p.l3); ++k)
                    for (int c = 0; c < mp / 4; ++c) {
                        const int base = loff[pi] + 16 * mp * k;
                        const std::string at = "TSW(" + std::to_string(4 * c) + " + usub, row)";
                        if (4 * c + 3 >= p.mul_in)
                            o("d", k, " = MFMA(wa", c, ", (", 4 * c, " + usub < ", p.mul_in, ") ? lds[", base, " + ", at,
                              "] : (T)0, d", k, ");");
                        else
                            o("d", k, " = MFMA(wa", c, ", lds[", base, " + ", at, "], d", k, ");");
                    }
                o.ind--;
                o("}");
            }
            o("if (olive) {");
            o.ind++;
            for (int v = 0; v < 4; ++v) {
                std::string wo = f64 ? "(" + std::to_string(16 * wt + 4 * v) + " + usub)"
                                     : "(" + std::to_string(16 * wt + v) + " + 4 * usub)";
                std::string guard = 16 * wt + 15 >= ir.mul ? "if (" + wo + " < " + std::to_string(ir.mul) + ") " : "";
                for (int k = 0; k < n_of(ir.l); ++k) {
                    std::ostringstream dst;
                    dst << "orow[" << ooff << " + " << wo << " * " << n_of(ir.l) << " + " << k << "]";
                    if (add)
                        o(guard, dst.str(), " += d", k, "[", v, "];");
                    else if (acc_variant)
                        o(guard, "{ if (acc) ", dst.str(), " += d", k, "[", v, "]; else ", dst.str(), " = d", k, "[", v, "]; }");
                    else
                        o(guard, dst.str(), " = d", k, "[", v, "];");
                }
            }
            o.ind--;
            o("}");
            o.ind--;
            o("}");
        }
    }
    o.ind--;
    o("}");
    o("");
}

int uvc_lds_elems(const Plan &P)
{
    int m = 1;
    for (const Group &g : P.uvc_groups) {
        int e = 0;
        for (int pi : g.paths) e += 16 * uvc_mu_pad(P.paths[pi]) * n_of(P.paths[pi].l3);
        m = std::max(m, e);
    }
    return m;
}

void emit_uvc_kernel(Out &o, const Plan &P)
{
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi) emit_uvc_group(o, P, gi);
    o("// one workgroup of ", 16 / P.uvc_rpw, " waves per 16 receivers; `group` selects the path group (launched in order)");
    o("extern \"C\" __global__ void __launch_bounds__(", 1024 / P.uvc_rpw, ", ", P.uvc_waves_per_eu,
      ") cgtp_conv_uvw(const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, T* __restrict__ out, long nrows, "
      "const int* __restrict__ order, int group)");
    o("{");
    o.ind++;
    o("__shared__ T lds[", uvc_lds_elems(P), "];  // T of the tile's 16 receivers, [p,k][u][row] (rows swizzled)");
    o("const long tile = blockIdx.x;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi)
        o("case ", gi, ": uvc_g", gi, "(tile, wv, lane, row_ptr, col, x, y, w, out, nrows, order, lds); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// The uvw convolution forward with a runtime `acc` (0: write the output as the forward does; 1:
// add to it), for the double backward's d/dgrad_out, a sum of three such convolutions.
void emit_uvc_acc_kernel(Out &o, const Plan &P)
{
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi) emit_uvc_group(o, P, gi, 1);
    o("extern \"C\" __global__ void __launch_bounds__(", 1024 / P.uvc_rpw, ", ", P.uvc_waves_per_eu,
      ") cgtp_conv_uvw_acc(const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, T* __restrict__ out, long nrows, "
      "const int* __restrict__ order, int group, int acc)");
    o("{");
    o.ind++;
    o("__shared__ T lds[", uvc_lds_elems(P), "];  // T of the tile's 16 receivers, [p,k][u][row] (rows swizzled)");
    o("const long tile = blockIdx.x;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi)
        o("case ", gi, ": uvca_g", gi, "(tile, wv, lane, row_ptr, col, x, y, w, out, nrows, order, lds, acc); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// The uvw convolution with radially projected weights, one radial channel per launch: the edge's
// SH values enter scaled by rho[e][rr] and the mixing uses Theta's row rr as W (by linearity the
// sum over rr of these launches is the convolution with W_e = rho_e Theta, whose per-edge blocks
// are never formed); `acc` as in cgtp_conv_uvw_acc.
void emit_uvc_rad_kernel(Out &o, const Plan &P)
{
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi) emit_uvc_group(o, P, gi, 2);
    o("extern \"C\" __global__ void __launch_bounds__(", 1024 / P.uvc_rpw, ", ", P.uvc_waves_per_eu,
      ") cgtp_conv_uvw_rad(const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, T* __restrict__ out, long nrows, "
      "const int* __restrict__ order, int group, int acc, const T* __restrict__ rho, int nrad, int rr)");
    o("{");
    o.ind++;
    o("__shared__ T lds[", uvc_lds_elems(P), "];  // T of the tile's 16 receivers, [p,k][u][row] (rows swizzled)");
    o("const long tile = blockIdx.x;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi)
        o("case ", gi, ": uvcr_g", gi, "(tile, wv, lane, row_ptr, col, x, y, w, out, nrows, order, lds, acc, rho, nrad, rr); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

// ------------------------------------------------------------------------------------------
// uvw batched backward (every mul_in, mul_out <= 16).  One wave per 16-row block; lane l works
// on row l % 16.  With G_p[row][u][k] = sum_w W_p[u][w] g[row][w][k] (MFMA: A = W_p[u = l%16][w],
// B = g[row = l%16][w][k], the lane ending with u = U(v) of its row):
//   dx[row][u][i] = sum_p sum_k A_p[i][k] G_p[row][u][k],  A_p[i][k] = sum_j C_ijk y[row][j]
//   dy[row][j]    = sum_p sum_{u,i,k} C_ijk x[row][u][i] G_p[row][u][k]
// (cgtp_tp_uvw_bwd_xy, one launch per input block; dY summed over the launches in order), and
//   dW_p[u][w] = sum_rows sum_k t_p[row][u][k] g[row][w][k],  t_p = sum_i A_p[i][k] x[row][u][i]
// as per-chunk MFMA partials over row blocks (t transposed through LDS so that the rows are the
// MFMA K dimension), summed in chunk order by cgtp_reduce_chunks.
// Row stride of the dY rows staged in LDS by the dx/dY pass: odd, so that the 16 lanes adding one
// component for their 16 rows hit 16 different banks (a stride of d_sh = 64 put them all on one).
int uvb_dy_stride(const Plan &P) { return P.d_sh | 1; }

// LDS words of the dx/dY kernel: the four waves' dY rows, then one [16][16 (2 l1 + 1) + 1] block
// per half of a split input block
int uvb_part_words(const Plan &P, int gi)
{
    const Group &g = P.uvb_x_groups[gi];
    return g.part ? 16 * (16 * (2 * P.ins[P.paths[g.paths[0]].i1].l + 1) + 1) : 0;
}
int uvb_part_offset(const Plan &P, int gi)
{
    int off = 4 * 16 * uvb_dy_stride(P);
    for (int k = 0; k < gi; ++k) off += uvb_part_words(P, k);
    return off;
}

std::string uvb_u(bool f64, int v) { return f64 ? "(usub + " + std::to_string(4 * v) + ")" : "(4 * usub + " + std::to_string(v) + ")"; }

void emit_uvb_xy_group(Out &o, const Plan &P, int gi)
{
    const Group &g = P.uvb_x_groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    Touch t = touched(P, g.paths);
    const int b1 = P.paths[g.paths[0]].i1;
    const Irrep &ir = P.ins[b1];
    const int n1 = n_of(ir.l);
    const int a = P.paths[g.paths[0]].a;
    o("__device__ __forceinline__ void uvbx_g", gi, "(long blk, int wv, int lane, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, const T* __restrict__ g, T* __restrict__ dx, "
      "T* __restrict__ dy, long nrows, T* dyl)");
    o("{");
    o.ind++;
    o("const int rl = lane & 15;");
    o("const int usub = lane >> 4;");
    o("const long row = blk * 16 + rl;");
    o("const bool live = row < nrows;");
    o("const long rr = live ? row : nrows - 1;  // rows past the end read row nrows-1 and store nothing");
    o("T* dyw = dyl + wv * ", 16 * uvb_dy_stride(P), ";  // this wave's dY rows (zeroed by the kernel)");
    for (int v = 0; v < 4; ++v) {
        const std::string u = uvb_u(f64, v);
        for (int i = 0; i < n1; ++i) {
            o("const T x", v, "_", i, " = ", u, " < ", ir.mul, " ? x[(size_t)rr * DX + ", a, " + (", u, " < ", ir.mul, " ? ", u,
              " : 0) * ", n1, " + ", i, "] : (T)0;");
            o("T d", v, "_", i, " = (T)0;");
        }
    }
    // The (path, k) blocks in order, software-pipelined: block b issues the MFMAs of block b + 1's
    // G (independent of its own) before its VALU work on G_b, so the MFMA chain runs under that
    // work instead of stalling it; gradient values are loaded PF blocks ahead (a ring of PF + 1
    // register sets) and the W operands one path ahead (two sets, by path parity).  Loads are
    // unconditional (clamped addresses) and masked where they are used: a load under a branch,
    // or a select right after it, made the compiler wait for it at once.
    std::vector<std::pair<int, int>> blocks;  // (index into g.paths, k)
    for (int q = 0; q < (int)g.paths.size(); ++q) {
        std::set<int> ks;
        for (const Nonzero &z : P.paths[g.paths[q]].nz) ks.insert(z.k);
        for (int k : ks) blocks.push_back({q, k});
    }
    const int nb = (int)blocks.size();
    const int PF = std::max(1, P.uvb_xy_prefetch), RS = PF + 1;
    auto wch_of = [&](int q) { return (P.paths[g.paths[q]].mul_out + 3) / 4; };
    auto load_g = [&](int bi) {
        const Path &p = P.paths[g.paths[blocks[bi].first]];
        const int k = blocks[bi].second, n3 = n_of(p.l3);
        for (int c = 0; c < wch_of(blocks[bi].first); ++c) {
            const std::string wv = 4 * c + 3 < p.mul_out ? std::to_string(4 * c) + " + usub"
                                                          : "(" + std::to_string(4 * c) + " + usub < " + std::to_string(p.mul_out) +
                                                                " ? " + std::to_string(4 * c) + " + usub : 0)";
            o("gs", bi % RS, "_", c, " = g[(size_t)rr * DOUT + ", p.o, " + (", wv, ") * ", n3, " + ", k, "];");
        }
    };
    // A operands of G: W_p[u = lane % 16][w = 4c + lane / 16] (rows and columns clamped)
    auto load_w = [&](int q) {
        const Path &p = P.paths[g.paths[q]];
        for (int c = 0; c < wch_of(q); ++c)
            o("wa", q % 2, "_", c, " = w[", p.w_off, " + (rl < ", p.mul_in, " ? rl : 0) * ", p.mul_out, " + (", 4 * c, " + usub < ",
              p.mul_out, " ? ", 4 * c, " + usub : 0)];");
    };
    auto issue_g = [&](int bi) {
        const int q = blocks[bi].first;
        const Path &p = P.paths[g.paths[q]];
        o("G", bi, " = (V4){0, 0, 0, 0};");
        for (int c = 0; c < wch_of(q); ++c) {
            std::string wa = "wa" + std::to_string(q % 2) + "_" + std::to_string(c);
            std::string gs = "gs" + std::to_string(bi % RS) + "_" + std::to_string(c);
            const std::string wok = "(" + std::to_string(4 * c) + " + usub < " + std::to_string(p.mul_out) + ")";
            if (p.mul_in < 16 || 4 * c + 3 >= p.mul_out)
                wa = "((rl < " + std::to_string(p.mul_in) + " && " + wok + ") ? " + wa + " : (T)0)";
            if (4 * c + 3 >= p.mul_out) gs = "(" + wok + " ? " + gs + " : (T)0)";
            o("G", bi, " = MFMA(", wa, ", ", gs, ", G", bi, ");");
        }
    };
    for (int set = 0; set < RS; ++set)
        for (int c = 0; c < 4; ++c) o("T gs", set, "_", c, " = (T)0;");
    for (int set = 0; set < 2; ++set)
        for (int c = 0; c < 4; ++c) o("T wa", set, "_", c, " = (T)0;");
    for (int bi = 0; bi < nb; ++bi) o("V4 G", bi, ";");
    if (nb > 0) {
        load_w(0);
        if (g.paths.size() > 1) load_w(1);
        for (int b = 0; b < std::min(PF, nb); ++b) load_g(b);
        issue_g(0);
    }
    int bi = 0;
    for (int q = 0; q < (int)g.paths.size(); ++q) {
        const Path &p = P.paths[g.paths[q]];
        const int n2 = n_of(p.l2);
        o("{");
        o.ind++;
        // this path's SH block, read here (an L1 hit after the first path of the row block):
        // holding every block for the whole group took 64 registers at l <= 7 and spilled (52 and
        // 148 bytes per lane for l1 = 6, 7; 0 and 20 this way, same time).  The opaque zero
        // offset keeps the compiler from merging these reads across paths.
        o("int zo = 0;");
        o("asm volatile(\"\" : \"+v\"(zo));");
        for (int j = 0; j < n2; ++j) o("const T y", p.i2, "_", j, " = y[(size_t)rr * DSH + zo + ", p.b + j, "];");
        for (int j = 0; j < n2; ++j) o("T h", j, " = (T)0;");
        // the wave's dY row values this path adds to, read now: the add at the path's end then
        // finds them in registers instead of waiting for an LDS read (the wave alone writes these
        // rows, and its LDS accesses complete in issue order, after the previous path's writes)
        for (int j = 0; j < n2; ++j) o("const T dyo", j, " = dyw[rl * ", uvb_dy_stride(P), " + ", p.b + j, "];");
        std::map<int, std::map<int, std::vector<const Nonzero *>>> byki;  // k -> i -> nonzeros
        for (const Nonzero &z : p.nz) byki[z.k][z.i].push_back(&z);
        for (auto &kk : byki) {
            o("{");
            o.ind++;
            if (bi + PF < nb) load_g(bi + PF);
            // the loads first: left alone the scheduler moves them below this block's MFMAs
            o("__builtin_amdgcn_sched_barrier(0);");
            if (bi + 1 < nb) issue_g(bi + 1);
            for (auto &ii : kk.second) {
                const int i = ii.first;
                const auto &v = ii.second;
                std::ostringstream e;
                e << lit(v[0]->c, f64) << " * y" << p.i2 << "_" << v[0]->j;
                for (size_t n = 1; n < v.size(); ++n) {
                    std::ostringstream f;
                    f << "FMA(" << lit(v[n]->c, f64) << ", y" << p.i2 << "_" << v[n]->j << ", " << e.str() << ")";
                    e.str(f.str());
                }
                o("{");
                o.ind++;
                o("const T A = ", e.str(), ";");
                for (int vv = 0; vv < 4; ++vv) o("d", vv, "_", i, " = FMA(A, G", bi, "[", vv, "], d", vv, "_", i, ");");
                o("const T si = FMA(x0_", i, ", G", bi, "[0], FMA(x1_", i, ", G", bi, "[1], FMA(x2_", i, ", G", bi, "[2], x3_", i,
                  " * G", bi, "[3])));");
                for (const Nonzero *z : v) o("h", z->j, " = FMA(", lit(z->c, f64), ", si, h", z->j, ");");
                o.ind--;
                o("}");
            }
            ++bi;
            // one output component at a time: without this the loads and MFMAs of every k of the
            // path are issued together and all of their results stay live
            o("__builtin_amdgcn_sched_barrier(0);");
            o.ind--;
            o("}");
        }
        // this path's W set is free once its last G has been issued (one block ago): fetch the
        // W of the path after next into it
        if (q + 2 < (int)g.paths.size()) load_w(q + 2);
        // dY of this path: sum the row's four lanes, then lane usub == 0 adds into the wave's LDS rows
        for (int j = 0; j < n2; ++j) {
            o(xadd("h" + std::to_string(j), 16));
            o(xadd("h" + std::to_string(j), 32));
        }
        o("if (usub == 0) {");
        o.ind++;
        for (int j = 0; j < n2; ++j) o("dyw[rl * ", uvb_dy_stride(P), " + ", p.b + j, "] = dyo", j, " + h", j, ";");
        o.ind--;
        o("}");
        // The dx sums are only read by the conditional store at the end; left alone the compiler
        // sinks every update there and keeps each (path, k) result of G live until then.  An
        // empty asm consumes and redefines them here, so each path's updates happen in place.
        for (int v = 0; v < 4; ++v)
            for (int i = 0; i < n1; ++i) o("asm volatile(\"\" : \"+v\"(d", v, "_", i, "));");
        o("__builtin_amdgcn_sched_barrier(0);");
        o.ind--;
        o("}");
    }
    if (g.part) {
        // one half of a split input block: its dx partial goes to the group's LDS rows (row r,
        // column u (2 l1 + 1) + i), which the kernel adds to the other half's after its barrier
        const int off = uvb_part_offset(P, gi);
        for (int v = 0; v < 4; ++v) {
            const std::string u = uvb_u(f64, v);
            for (int i = 0; i < n1; ++i)
                o("dyl[", off, " + rl * ", 16 * n1 + 1, " + ", u, " * ", n1, " + ", i, "] = d", v, "_", i, ";");
        }
    }
    o("if (live && dx) {");
    o.ind++;
    for (int v = 0; v < 4 && !g.part; ++v) {
        const std::string u = uvb_u(f64, v);
        o("if (", u, " < ", ir.mul, ") {");
        o.ind++;
        for (int i = 0; i < n1; ++i) o("dx[(size_t)rr * DX + ", a, " + ", u, " * ", n1, " + ", i, "] = d", v, "_", i, ";");
        o.ind--;
        o("}");
    }
    if (gi == 0) {
        // input blocks that no path uses get zero gradients
        int off = 0;
        for (int b = 0; b < (int)P.ins.size(); ++b) {
            bool used = false;
            for (const Path &q : P.paths) used = used || q.i1 == b;
            if (!used) o("for (int c = lane >> 4; c < ", P.ins[b].dim(), "; c += 4) dx[(size_t)rr * DX + ", off, " + c] = (T)0;");
            off += P.ins[b].dim();
        }
    }
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    o("");
}

// Gradient staging of the dW kernel: the block g[16 rows][slot of path p] (S = mul_out (2 l3 + 1)
// values per row, contiguous in memory) is loaded whole, `cp` consecutive columns of 64 / cp rows
// per load instruction (so that each instruction reads whole lines), and written to LDS rows of
// stride T, T = 16 (mod 32): the MFMA B reads (16 channels at stride 2 l3 + 1, odd, times two rows
// T apart) then fall on distinct banks.
struct UvbStage {
    int S, cp, rp, ncol, loads, T;
};
UvbStage uvb_stage(const Path &p)
{
    UvbStage st;
    st.S = p.mul_out * n_of(p.l3);
    st.cp = st.S > 16 ? 32 : 16;
    st.rp = 64 / st.cp;
    st.ncol = (st.S + st.cp - 1) / st.cp;
    st.loads = (16 / st.rp) * st.ncol;
    st.T = (st.cp * st.ncol + 15) / 32 * 32 + 16;
    return st;
}
int uvb_stage_words(const Plan &P, const Group &g)
{
    int w = 0;
    for (int pi : g.paths) w = std::max(w, 16 * uvb_stage(P.paths[pi]).T);
    return w;
}
int uvb_stage_words(const Plan &P)
{
    int w = 0;
    for (const Group &g : P.uvb_w_groups) w = std::max(w, uvb_stage_words(P, g));
    return w;
}

void emit_uvb_w_group(Out &o, const Plan &P, int gi)
{
    const Group &g = P.uvb_w_groups[gi];
    const bool f64 = P.dtype == CGTP_F64;
    Touch t = touched(P, g.paths);
    o("__device__ __forceinline__ void uvbw_g", gi, "(long chunk, int wv, int lane, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ g, T* __restrict__ ws, long nrows, long nblocks, long bpc, T* tl)");
    o("{");
    o.ind++;
    o("const int rl = lane & 15;");
    o("const int usub = lane >> 4;");
    // this wave's transpose tile [row][u], u XOR row inside each row: the write (16 rows x 4 u) and
    // the read (4 rows x 16 u) each touch distinct banks (rows padded to 17 left 2-way conflicts)
    // With the pipeline on, two tiles per wave: block b writes its t into tile b % 2 and, at its
    // start, reads the tile block b - 1 wrote, whose MFMAs it issues after its own VALU work, so
    // that the LDS round trip and the MFMA chain run under that work instead of stalling the wave.
    const bool pipe = P.uvb_w_pipeline;
    const bool gst = P.uvb_w_stage;
    o("T* tw = tl + wv * ", pipe ? 512 : 256, ";");
    if (gst) o("T* gb = tl + ", 4 * (pipe ? 512 : 256), " + wv * ", uvb_stage_words(P), ";  // this wave's staged gradient block");
    for (int pi : g.paths) o("V4 D", pi, " = {0, 0, 0, 0};");
    o("const long b0 = chunk * bpc;");
    o("const long b1 = b0 + bpc < nblocks ? b0 + bpc : nblocks;");
    std::map<int, std::vector<int>> by_i1;
    for (int pi : g.paths) by_i1[P.paths[pi].i1].push_back(pi);
    // Every load a row block needs is issued one step ahead: its y and the x of its first input
    // block during the previous row block, the x of each later input block during the one
    // before it, and the gradient values of its first (path, k) block during the previous row
    // block's last one (one wave per SIMD: nothing else covers their latency).
    auto y_loads = [&](const std::string &dst, const std::string &rrx) {
        for (int b : t.i2) {
            int off = 0;
            for (int bb = 0; bb < b; ++bb) off += P.sh[bb].dim();
            for (int j = 0; j < n_of(P.sh[b].l); ++j)
                o(dst, b, "_", j, " = y[(size_t)", rrx, " * DSH + ", off + j, "];");
        }
    };
    auto x_loads = [&](int i1, const std::string &rrx, bool declare = false) {
        const std::string Ty = declare ? "const T " : "";
        const Irrep &ir = P.ins[i1];
        const int n1 = n_of(ir.l);
        const int a = P.paths[by_i1[i1][0]].a;
        // x in the forward's layout: lane holds u = 4c + lane / 16.  Every load of this kernel is
        // unconditional, from an element that exists (rows and channels clamped), and the
        // masking waits for the use: a load under a branch made the compiler's wait counting
        // fall back to waiting for every load in flight, and a select right after the load
        // waits for it there; either defeated the prefetching below.
        for (int c = 0; c < 4; ++c)
            for (int i = 0; i < n1; ++i) {
                if (4 * c + 3 < ir.mul)
                    o(Ty, "xp", c, "_", i, " = x[(size_t)", rrx, " * DX + ", a, " + (", 4 * c, " + usub) * ", n1, " + ", i, "];");
                else
                    o(Ty, "xp", c, "_", i, " = x[(size_t)", rrx, " * DX + ", a, " + (", 4 * c, " + usub < ", ir.mul, " ? ", 4 * c,
                      " + usub : 0) * ", n1, " + ", i, "];");
            }
    };
    // the (path, k) blocks in emission order; each block loads the next one's B operands (the
    // gradient values of its four row groups) before its own work, so that their latency is
    // covered by the block (one wave per SIMD leaves nothing else to hide it)
    std::vector<std::pair<int, int>> blocks;
    for (auto &kv : by_i1)
        for (int pi : kv.second) {
            std::set<int> ks;
            for (const Nonzero &z : P.paths[pi].nz) ks.insert(z.k);
            for (int k : ks) blocks.push_back({pi, k});
        }
    // gradient values of block bi of the row block starting at row `rb` (a variable name), into
    // register set `set`
    auto load_g = [&](size_t bi, const std::string &rb, int set) {
        const Path &p = P.paths[blocks[bi].first];
        const int k = blocks[bi].second, n3 = n_of(p.l3);
        for (int m = 0; m < 4; ++m) {
            o("{");
            o.ind++;
            o("const long br = ", rb, " * 16 + ", 4 * m, " + usub;");
            o("gp", set, "_", m, " = g[(size_t)(br < nrows ? br : nrows - 1) * DOUT + ", p.o, " + (rl < ", p.mul_out,
              " ? rl : 0) * ", n3, " + ", k, "];");
            o.ind--;
            o("}");
        }
    };
    // The gradient values run D blocks ahead in a ring of D register sets (a block's own work is
    // a few hundred cycles, a gradient load under load a thousand or more).  The block stream of
    // a row block is padded with D - 1 at most load-only steps to a multiple of D, so that block
    // b always uses set b % D, also across row blocks.
    const int nbk = (int)blocks.size();
    const int D = std::max(1, P.uvb_w_prefetch);
    const int padded = nbk == 0 ? 0 : (nbk + D - 1) / D * D;
    // the load issued at stream position `pos` (consuming nothing at pad positions): block pos + D
    auto ahead = [&](int pos) {
        const int tgt = pos + D;
        if (tgt < nbk) {
            load_g((size_t)tgt, "blk", tgt % D);
        } else if (tgt >= padded) {
            load_g((size_t)(tgt - padded), "(blk + 1)", tgt % D);  // past the chunk: clamped, unused
        }
    };
    // staged mode: paths in emission order; each path's block is loaded (into gr registers) while
    // the path before it computes, and written to LDS where the path starts
    std::vector<int> porder;
    for (auto &kv : by_i1)
        for (int pi : kv.second) porder.push_back(pi);
    int gr_max = 0;
    for (int pi : g.paths) gr_max = std::max(gr_max, uvb_stage(P.paths[pi]).loads);
    auto stage_load = [&](int pi, const std::string &rb) {
        const Path &p = P.paths[pi];
        const UvbStage st = uvb_stage(p);
        const int lsh = st.cp == 32 ? 5 : 4;
        // one (wave-uniform) base per row block and unsigned 32-bit offsets from it; rows past the
        // end read row nrows - 1 (rb is a block of the tensor: rb * 16 <= nrows - 1)
        o("{");
        o.ind++;
        o("const T* gs = g + (size_t)(", rb, ") * 16 * DOUT + ", p.o, ";");
        o("const unsigned lim = (unsigned)(nrows - 1 - (", rb, ") * 16);");
        for (int r = 0; r < 16 / st.rp; ++r) {
            o("{");
            o.ind++;
            o("const unsigned sr = ", st.rp * r, "u + (lane >> ", lsh, ") < lim ? ", st.rp * r, "u + (lane >> ", lsh, ") : lim;");
            for (int c = 0; c < st.ncol; ++c) {
                const std::string col = std::to_string(st.cp * c) + " + (lane & " + std::to_string(st.cp - 1) + ")";
                const std::string cl = st.cp * (c + 1) > st.S ? "(" + col + " < " + std::to_string(st.S) + " ? " + col + " : " +
                                                                   std::to_string(st.S - 1) + ")"
                                                             : "(" + col + ")";
                o("gr", r * st.ncol + c, " = gs[sr * (unsigned)DOUT + (unsigned)", cl, "];");
            }
            o.ind--;
            o("}");
        }
        o.ind--;
        o("}");
    };
    auto stage_store = [&](int pi) {
        const UvbStage st = uvb_stage(P.paths[pi]);
        const int lsh = st.cp == 32 ? 5 : 4;
        for (int r = 0; r < 16 / st.rp; ++r)
            for (int c = 0; c < st.ncol; ++c)
                o("gb[(", st.rp * r, " + (lane >> ", lsh, ")) * ", st.T, " + ", st.cp * c, " + (lane & ", st.cp - 1, ")] = gr",
                  r * st.ncol + c, ";");
    };
    int n1max = 1;
    for (auto &kv : by_i1) n1max = std::max(n1max, n_of(P.ins[kv.first].l));
    // The staged blocks take 64 registers per lane at l = 7; to make room, that mode reads each
    // path's SH block where the path starts (L1 hits after the row block's first path) instead of
    // holding every block and the next row block's, and loads x where its section starts.
    if (!gst) {
        for (int b : t.i2)
            for (int j = 0; j < n_of(P.sh[b].l); ++j) o("T yp", b, "_", j, " = (T)0;");
        for (int c = 0; c < 4; ++c)
            for (int i = 0; i < n1max; ++i) o("T xp", c, "_", i, " = (T)0;");
    }
    if (gst)
        for (int i = 0; i < gr_max; ++i) o("T gr", i, " = (T)0;");
    else
        for (int set = 0; set < D; ++set)
            for (int m = 0; m < 4; ++m) o("T gp", set, "_", m, " = (T)0;");
    if (pipe)
        for (int par = 0; par < 2; ++par)
            for (int m = 0; m < 4; ++m) o("T gq", par, "_", m, " = (T)0;");
    o("if (b0 < b1) {");
    o.ind++;
    o("const long row0 = b0 * 16 + rl;");
    o("const long rr0 = row0 < nrows ? row0 : nrows - 1;");
    if (!gst) {
        y_loads("yp", "rr0");
        if (!by_i1.empty()) x_loads(by_i1.begin()->first, "rr0");
    }
    if (gst) {
        if (!porder.empty()) stage_load(porder[0], "b0");
    } else {
        for (int b = 0; b < std::min(D, nbk); ++b) load_g((size_t)b, "b0", b % D);
    }
    o.ind--;
    o("}");
    o("for (long blk = b0; blk < b1; ++blk) {");
    o.ind++;
    o("const long row = blk * 16 + rl;");
    o("const bool live = row < nrows;");
    o("const long rr = live ? row : nrows - 1;");
    o("const bool more = blk + 1 < b1;");
    o("const long rowx = (blk + 1) * 16 + rl;");
    o("const long rrx = more ? (rowx < nrows ? rowx : nrows - 1) : rr;");
    if (!gst) {
        for (int b : t.i2)
            for (int j = 0; j < n_of(P.sh[b].l); ++j) o("const T y", b, "_", j, " = yp", b, "_", j, ";");
        y_loads("yp", "rrx");  // rrx = rr after the last row block: loaded again, unused
    }
    size_t bidx = 0;
    size_t sec = 0;
    int prev_pi = -1, par = 0;  // pipeline: the block whose MFMAs are pending, and this block's tile
    // MFMAs of the pending block: A = t[row = 4m + lane/16][u = lane%16] from its tile
    auto pending_mfma = [&](const std::string &ta) {
        for (int m = 0; m < 4; ++m)
            o("D", prev_pi, " = MFMA(", ta, m, ", gq", par ^ 1, "_", m, ", D", prev_pi, ");");
    };
    auto tile_read = [&](int tile, int m) {
        return "tw[" + std::to_string(tile * 256 + 64 * m) + " + usub * 16 + (rl ^ (" + std::to_string(4 * m) + " + usub))]";
    };
    for (auto &kv : by_i1) {
        const Irrep &ir = P.ins[kv.first];
        const int n1 = n_of(ir.l);
        o("{");
        o.ind++;
        if (gst) x_loads(kv.first, "rr", true);
        for (int c = 0; c < 4; ++c)
            for (int i = 0; i < n1; ++i) {
                if (4 * c + 3 < ir.mul)
                    o("const T x", c, "_", i, " = xp", c, "_", i, ";");
                else
                    o("const T x", c, "_", i, " = ", 4 * c, " + usub < ", ir.mul, " ? xp", c, "_", i, " : (T)0;");
            }
        // the next input block's x: this row block's, or the next row block's first
        if (gst) {
        } else if (++sec < by_i1.size()) {
            x_loads(std::next(by_i1.begin(), (long)sec)->first, "rr");
        } else {
            x_loads(by_i1.begin()->first, "rrx");
        }
        for (int pi : kv.second) {
            const Path &p = P.paths[pi];
            std::map<int, std::map<int, std::vector<const Nonzero *>>> byki;
            for (const Nonzero &z : p.nz) byki[z.k][z.i].push_back(&z);
            const UvbStage st = uvb_stage(p);
            o("{");
            o.ind++;
            if (gst) {
                // opaque zero offset: keeps the compiler from merging these reads across paths
                int off = 0;
                for (int bb = 0; bb < p.i2; ++bb) off += P.sh[bb].dim();
                o("int zo = 0;");
                o("asm volatile(\"\" : \"+v\"(zo));");
                for (int j = 0; j < n_of(p.l2); ++j) o("const T y", p.i2, "_", j, " = y[(size_t)rr * DSH + zo + ", off + j, "];");
                // this path's gradient block into LDS (the reads of the path before it are
                // issued, and the wave's LDS accesses complete in order), then the next path's
                // loads: that of the next row block after the last path (clamped past the end)
                const size_t at = (size_t)(std::find(porder.begin(), porder.end(), pi) - porder.begin());
                o("WAVE_SYNC();");
                stage_store(pi);
                if (at + 1 < porder.size())
                    stage_load(porder[at + 1], "blk");
                else
                    stage_load(porder[0], "(blk + 1 < b1 ? blk + 1 : blk)");  // the chunk's last: loaded again, unused
                o("WAVE_SYNC();");
            }
            for (auto &kk : byki) {
                o("{");
                o.ind++;
                // gradient values of rows past the end and of channels past mul_out are zero
                const bool wmask = P.paths[pi].mul_out < 16;
                if (pipe) {
                    // the pending block's t, read before this block's work (pinned here)
                    o("WAVE_SYNC();");
                    if (prev_pi >= 0) {
                        for (int m = 0; m < 4; ++m) o("const T ta", m, " = ", tile_read(par ^ 1, m), ";");
                        o("__builtin_amdgcn_sched_barrier(0);");
                    }
                }
                for (int m = 0; m < 4; ++m) {
                    const std::string src =
                        gst ? "gb[" + std::to_string(4 * m * st.T) + " + usub * " + std::to_string(st.T) + " + " +
                                  (wmask ? "(rl < " + std::to_string(p.mul_out) + " ? rl : 0)" : std::string("rl")) + " * " +
                                  std::to_string(n_of(p.l3)) + " + " + std::to_string(kk.first) + "]"
                            : "gp" + std::to_string((int)bidx % D) + "_" + std::to_string(m);
                    o(pipe ? "gq" + std::to_string(par) + "_" : std::string("const T gc"), m, " = (blk * 16 + ", 4 * m, " + usub < nrows",
                      wmask ? " && rl < " + std::to_string(P.paths[pi].mul_out) : std::string(), ") ? ", src, " : (T)0;");
                }
                if (!gst) ahead((int)bidx);
                ++bidx;
                for (auto &ii : kk.second) {
                    const auto &v = ii.second;
                    std::ostringstream e;
                    e << lit(v[0]->c, f64) << " * y" << p.i2 << "_" << v[0]->j;
                    for (size_t n = 1; n < v.size(); ++n) {
                        std::ostringstream f;
                        f << "FMA(" << lit(v[n]->c, f64) << ", y" << p.i2 << "_" << v[n]->j << ", " << e.str() << ")";
                        e.str(f.str());
                    }
                    o("const T A", ii.first, " = ", e.str(), ";");
                }
                if (!pipe) o("WAVE_SYNC();");
                for (int c = 0; c < 4; ++c) {
                    std::ostringstream e;
                    bool first = true;
                    for (auto &ii : kk.second) {
                        if (first) {
                            e << "A" << ii.first << " * x" << c << "_" << ii.first;
                            first = false;
                        } else {
                            std::ostringstream f;
                            f << "FMA(A" << ii.first << ", x" << c << "_" << ii.first << ", " << e.str() << ")";
                            e.str(f.str());
                        }
                    }
                    o("tw[", pipe ? par * 256 : 0, " + rl * 16 + ((", 4 * c, " + usub) ^ rl)] = live ? ", e.str(), " : (T)0;");
                }
                if (pipe) {
                    if (prev_pi >= 0) pending_mfma("ta");
                    prev_pi = pi;
                    par ^= 1;
                } else {
                    o("WAVE_SYNC();");
                    // rows are the MFMA K dimension: A = t[row = 4m + lane/16][u = lane%16], B = g[row][w = lane%16][k]
                    for (int m = 0; m < 4; ++m) o("D", pi, " = MFMA(", tile_read(0, m), ", gc", m, ", D", pi, ");");
                }
                o("__builtin_amdgcn_sched_barrier(0);");
                o.ind--;
                o("}");
            }
            o.ind--;
            o("}");  // path
        }
        o.ind--;
        o("}");
    }
    if (!gst)
        for (int pos = nbk; pos < padded; ++pos) ahead(pos);  // load-only steps of the padding
    if (pipe && prev_pi >= 0) {
        // the row block's last block
        o("{");
        o.ind++;
        o("WAVE_SYNC();");
        for (int m = 0; m < 4; ++m) o("const T ta", m, " = ", tile_read(par ^ 1, m), ";");
        pending_mfma("ta");
        o("WAVE_SYNC();");
        o.ind--;
        o("}");
    }
    o.ind--;
    o("}");  // row blocks
    // lane holds D[u = U(v)][w = lane % 16]
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        for (int v = 0; v < 4; ++v) {
            const std::string u = uvb_u(f64, v);
            o("if (", u, " < ", p.mul_in, " && rl < ", p.mul_out, ") ws[(size_t)chunk * WN + ", p.w_off, " + ", u, " * ", p.mul_out,
              " + rl] = D", pi, "[", v, "];");
        }
    }
    o.ind--;
    o("}");
    o("");
}

// out[i] = sum over chunks of ws[chunk][i] (nchunks = 0 writes zeros).  One workgroup of 16
// waves per 64 consecutive i: wave v sums the v-th contiguous sixteenth of the chunks in chunk
// order (eight loads in flight), then wave 0 adds the sixteen partials in wave order; the order
// of every sum is fixed by nchunks alone.
void emit_reduce_chunks(Out &o)
{
    o("extern \"C\" __global__ void __launch_bounds__(1024) cgtp_reduce_chunks(const T* __restrict__ ws, long nchunks, "
      "T* __restrict__ out)");
    o("{");
    o.ind++;
    o("__shared__ T part[16 * 64];");
    o("const int lane = threadIdx.x & 63;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const long i = (long)blockIdx.x * 64 + lane;");
    o("const bool ok = i < WN;");
    o("const long per = (nchunks + 15) / 16;");
    o("const long c0 = wv * per;");
    o("const long c1 = c0 + per < nchunks ? c0 + per : nchunks;");
    o("const T* p = ws + (ok ? i : 0);");
    o("T s = (T)0;");
    o("long c = c0;");
    o("for (; ok && c + 8 <= c1; c += 8) {");
    o.ind++;
    o("T v[8];");
    o("for (int k = 0; k < 8; ++k) v[k] = p[(size_t)(c + k) * WN];");
    o("for (int k = 0; k < 8; ++k) s += v[k];");
    o.ind--;
    o("}");
    o("for (; ok && c < c1; ++c) s += p[(size_t)c * WN];");
    o("part[wv * 64 + lane] = s;");
    o("__syncthreads();");
    o("if (wv == 0 && ok) {");
    o.ind++;
    o("T t = part[lane];");
    o("for (int v = 1; v < 16; ++v) t += part[v * 64 + lane];");
    o("out[i] = t;");
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    o("");
}

void emit_uvb_kernels(Out &o, const Plan &P)
{
    if (!P.uvb_ok) {
        o("// uvw batched backward not generated: some multiplicity exceeds 16");
        return;
    }
    o("#define WN ", P.w_numel, "L");
    o("#define WAVE_SYNC() do { __builtin_amdgcn_fence(__ATOMIC_RELEASE, \"wavefront\"); "
      "__builtin_amdgcn_wave_barrier(); __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, \"wavefront\"); } while (0)");
    for (int gi = 0; gi < (int)P.uvb_x_groups.size(); ++gi) emit_uvb_xy_group(o, P, gi);
    // One workgroup per 16-row block; its four waves share the input blocks (each wave its own
    // list, balanced by a cost estimate, heaviest first), write the dx of their blocks, and add
    // their dY rows in LDS; after the barrier the four waves' rows are summed in wave order.
    std::vector<std::pair<long, int>> cost;
    for (int gi = 0; gi < (int)P.uvb_x_groups.size(); ++gi) {
        long c = 0;
        for (int pi : P.uvb_x_groups[gi].paths) {
            const Path &p = P.paths[pi];
            c += (long)p.nz.size() * 6 + 16L * n_of(p.l3);
        }
        cost.push_back({c, gi});
    }
    std::stable_sort(cost.begin(), cost.end(), [](auto &a, auto &b) { return a.first > b.first; });
    std::vector<std::vector<int>> lists(4);
    std::vector<long> load(4, 0);
    for (auto &cg : cost) {
        const int wv = (int)(std::min_element(load.begin(), load.end()) - load.begin());
        lists[wv].push_back(cg.second);
        load[wv] += cg.first;
    }
    o("extern \"C\" __global__ void __launch_bounds__(256, 1) cgtp_tp_uvw_bwd_xy(const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ w, const T* __restrict__ g, T* __restrict__ dx, "
      "T* __restrict__ dy, long nrows, long nblocks)");
    o("{");
    o.ind++;
    const int dsp = uvb_dy_stride(P);
    const int nx = (int)P.uvb_x_groups.size();
    const int lds_words = uvb_part_offset(P, nx);
    o("__shared__ T dyl[", lds_words, "];  // per wave 16 dY rows of stride ", dsp, ", then the dx halves of split input blocks");
    o("const long blk = blockIdx.x;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("for (int c = threadIdx.x; c < ", 4 * 16 * dsp, "; c += 256) dyl[c] = (T)0;");
    o("__syncthreads();");
    o("switch (wv) {");
    for (int wv = 0; wv < 4; ++wv) {
        o("case ", wv, ":");
        o.ind++;
        for (int gi : lists[wv]) o("uvbx_g", gi, "(blk, wv, lane, x, y, w, g, dx, dy, nrows, dyl);");
        o("break;");
        o.ind--;
    }
    o("default: break;");
    o("}");
    o("__syncthreads();");
    o("if (dy) {");
    o.ind++;
    o("for (int c = threadIdx.x; c < ", 16 * P.d_sh, "; c += 256) {");
    o.ind++;
    o("const long row = blk * 16 + c / DSH;");
    o("const int lc = (c / DSH) * ", dsp, " + c % DSH;");
    o("if (row < nrows) dy[(size_t)row * DSH + c % DSH] = ((dyl[lc] + dyl[", 16 * dsp, " + lc]) + dyl[", 32 * dsp,
      " + lc]) + dyl[", 48 * dsp, " + lc];");
    o.ind--;
    o("}");
    o.ind--;
    o("}");
    // dx of each split input block: first half + second half, stored by all 256 threads
    for (int gi = 0; gi + 1 < nx; ++gi) {
        const Group &h1 = P.uvb_x_groups[gi];
        if (h1.part != 1) continue;
        const Path &p0 = P.paths[h1.paths[0]];
        const Irrep &ir = P.ins[p0.i1];
        const int n1 = n_of(ir.l), cols = ir.mul * n1, rs = 16 * n1 + 1;
        const int o1 = uvb_part_offset(P, gi), o2 = uvb_part_offset(P, gi + 1);
        o("if (dx) {");
        o.ind++;
        o("for (int c = threadIdx.x; c < ", 16 * cols, "; c += 256) {");
        o.ind++;
        o("const int r = c / ", cols, ", col = c - r * ", cols, ";");
        o("const long row = blk * 16 + r;");
        o("if (row < nrows) dx[(size_t)row * DX + ", p0.a, " + col] = dyl[", o1, " + r * ", rs, " + col] + dyl[", o2, " + r * ", rs,
          " + col];");
        o.ind--;
        o("}");
        o.ind--;
        o("}");
    }
    o.ind--;
    o("}");
    o("");
    for (int gi = 0; gi < (int)P.uvb_w_groups.size(); ++gi) emit_uvb_w_group(o, P, gi);
    o("// one wave per (path group, chunk of row blocks), chunk-major within a group");
    o("extern \"C\" __global__ void __launch_bounds__(256, ", P.uvb_w_waves_per_eu, ") cgtp_tp_uvw_bwd_w(const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ g, T* __restrict__ ws, long nrows, long nblocks, long bpc, "
      "long nchunks, long nwaves)");
    o("{");
    o.ind++;
    o("__shared__ T tl[", 4 * (P.uvb_w_pipeline ? 512 : 256) + (P.uvb_w_stage ? 4 * uvb_stage_words(P) : 0), "];");
    o("const long wave = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("if (wave >= nwaves) return;");
    o("const int group = (int)(wave / nchunks);");
    o("const long chunk = wave - (long)group * nchunks;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.uvb_w_groups.size(); ++gi)
        o("case ", gi, ": uvbw_g", gi, "(chunk, wv, lane, x, y, g, ws, nrows, nblocks, bpc, tl); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
    emit_reduce_chunks(o);
}

// ------------------------------------------------------------------------------------------
// uvw convolution backward.  With the receiver-side products
//   G_p[n][u][k] = sum_w W_p[u][w] g[n][slot(p)][w][k]
// (cgtp_conv_uvw_bwd_g, MFMA per 16-receiver tile), the input and SH gradients are those of a
// uvu convolution with unit weights whose output has one block per path (mul_in(p) x l3): the
// sender pass of that internal plan reads G in place of the output gradient.  The weight
// gradient
//   dW_p[u][w] = sum_n sum_k T_p[n][u][k] g[n][slot(p)][w][k],
// T_p the unweighted per-receiver sums of the forward, reuses the forward's edge pass (T staged
// in LDS for the tile's 16 receivers), then contracts over the 16 receivers on MFMA with the
// receivers as the K dimension (A = T[u = lane % 16][row = 4m + lane / 16], B = g[row][w = lane %
// 16][k]); every tile writes its partial, and cgtp_reduce_chunks sums them in tile order.
// work items of the G kernel: (path, 16-channel block of u)
int ucb_items(const Plan &P, std::vector<std::pair<int, int>> *items)
{
    int n = 0;
    for (int pi = 0; pi < (int)P.paths.size(); ++pi)
        for (int ut = 0; ut * 16 < P.paths[pi].mul_in; ++ut, ++n)
            if (items) items->push_back({pi, ut});
    return n;
}

void emit_ucb_g_kernel(Out &o, const Plan &P)
{
    const bool f64 = P.dtype == CGTP_F64;
    std::vector<std::pair<int, int>> items;
    const int nitems = ucb_items(P, &items);
    std::vector<int> goff(P.paths.size());
    for (int pi = 0, acc = 0; pi < (int)P.paths.size(); ++pi) {
        goff[pi] = acc;
        acc += P.paths[pi].mul_in * n_of(P.paths[pi].l3);
    }
    o("// one wave per (16-receiver tile, path, 16-channel block of u), tile-major");
    o("extern \"C\" __global__ void __launch_bounds__(256) cgtp_conv_uvw_bwd_g(const T* __restrict__ w, "
      "const T* __restrict__ g, T* __restrict__ G, long nrows, long nwaves)");
    o("{");
    o.ind++;
    o("const long wave = (long)blockIdx.x * 4 + WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("if (wave >= nwaves) return;");
    o("const long tile = wave / ", nitems, ";");
    o("const int item = (int)(wave - tile * ", nitems, ");");
    o("const int usub = lane >> 4;");
    o("const int row = lane & 15;");
    o("const long n = tile * 16 + row;");
    o("const bool live = n < nrows;");
    o("const long nn = live ? n : nrows - 1;");
    o("switch (item) {");
    for (int it = 0; it < nitems; ++it) {
        const int q = P.paths[items[it].first].slot, ut = items[it].second;
        const Irrep &ir = P.out[q];
        const int n3 = n_of(ir.l);
        int ooff = 0;
        for (int qq = 0; qq < q; ++qq) ooff += P.out[qq].dim();
        const int cs = (ir.mul + 3) / 4;
        o("case ", it, ": {");
        o.ind++;
        const std::vector<int> ps = {items[it].first};
        // operands first (one wait for all of them): B = g[row = lane % 16][w = 4c + lane / 16][k]
        // for every k, A = W_p[u = 16 ut + lane % 16][w = 4c + lane / 16]
        for (int k = 0; k < n3; ++k)
            for (int c = 0; c < cs; ++c) {
                const std::string wv = "(" + std::to_string(4 * c) + " + usub)";
                if (4 * c + 3 >= ir.mul)
                    o("const T b", k, "_", c, " = ", wv, " < ", ir.mul, " ? g[(size_t)nn * DOUT + ", ooff, " + (", wv, " < ", ir.mul,
                      " ? ", wv, " : 0) * ", n3, " + ", k, "] : (T)0;");
                else
                    o("const T b", k, "_", c, " = g[(size_t)nn * DOUT + ", ooff, " + ", wv, " * ", n3, " + ", k, "];");
            }
        const std::string u = "(" + std::to_string(16 * ut) + " + row)";
        for (int pi : ps) {
            const Path &p = P.paths[pi];
            for (int c = 0; c < cs; ++c) {
                const std::string wv = "(" + std::to_string(4 * c) + " + usub)";
                if (16 * ut + 15 >= p.mul_in || 4 * c + 3 >= p.mul_out) {
                    const std::string ok = "(" + u + " < " + std::to_string(p.mul_in) + " && " + wv + " < " +
                                           std::to_string(p.mul_out) + ")";
                    o("const T a", pi, "_", c, " = ", ok, " ? w[", p.w_off, " + (", ok, " ? ", u, " * ", p.mul_out, " + ", wv,
                      " : 0)] : (T)0;");
                } else {
                    o("const T a", pi, "_", c, " = w[", p.w_off, " + ", u, " * ", p.mul_out, " + ", wv, "];");
                }
            }
        }
        for (int pi : ps)
            for (int k = 0; k < n3; ++k) {
                o("V4 d", pi, "_", k, " = {0, 0, 0, 0};");
                for (int c = 0; c < cs; ++c) o("d", pi, "_", k, " = MFMA(a", pi, "_", c, ", b", k, "_", c, ", d", pi, "_", k, ");");
            }
        // lane holds G[u = 16 ut + U(v)][row = lane % 16]; one branch for all stores, so that
        // the loads and MFMAs above form one scheduling region
        o("if (live) {");
        o.ind++;
        for (int pi : ps) {
            const Path &p = P.paths[pi];
            for (int k = 0; k < n3; ++k)
                for (int v = 0; v < 4; ++v) {
                    const std::string uu = "(" + std::to_string(16 * ut) + " + " + uvb_u(f64, v) + ")";
                    const std::string guard = 16 * ut + 15 >= p.mul_in ? "if (" + uu + " < " + std::to_string(p.mul_in) + ") " : "";
                    o(guard, "G[(size_t)n * DG + ", goff[pi], " + ", uu, " * ", n3, " + ", k, "] = d", pi, "_", k, "[", v, "];");
                }
        }
        o.ind--;
        o("}");
        o("break;");
        o.ind--;
        o("}");
    }
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
}

void emit_ucb_w_group(Out &o, const Plan &P, int gi)
{
    const Group &g = P.uvc_groups[gi];
    std::map<int, int> loff;
    int lds_elems = 0;
    for (int pi : g.paths) {
        loff[pi] = lds_elems;
        lds_elems += 16 * uvc_mu_pad(P.paths[pi]) * n_of(P.paths[pi].l3);
    }
    const bool f64 = P.dtype == CGTP_F64;
    const int nw = 16 / P.uvc_rpw;
    emit_tsw(o);
    o("__device__ __forceinline__ void ucw_g", gi,
      "(long tile, int wv, int lane, const int* __restrict__ row_ptr, const int* __restrict__ col, "
      "const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ g, T* __restrict__ ws, long nrows, "
      "const int* __restrict__ order, T* lds)");
    o("{");
    o.ind++;
    emit_uvc_phase_a(o, P, g, loff);
    o("__syncthreads();");
    o("const int usub = lane >> 4;");
    o("const int row = lane & 15;");
    // receivers of the B rows 4m + lane / 16
    for (int m = 0; m < 4; ++m) {
        o("const long bi", m, " = tile * 16 + ", 4 * m, " + usub;");
        o("const bool bl", m, " = bi", m, " < nrows;");
        o("const long bn", m, " = bl", m, " ? (order ? (long)order[bi", m, "] : bi", m, ") : 0;");
    }
    int item = 0;
    for (int pi : g.paths) {
        const Path &p = P.paths[pi];
        const int n3 = n_of(p.l3), mp = uvc_mu_pad(p);
        const int uts = (p.mul_in + 15) / 16, wts = (p.mul_out + 15) / 16;
        for (int wt = 0; wt < wts; ++wt, ++item) {
            o("if (wv == ", item % nw, ") {");
            o.ind++;
            for (int ut = 0; ut < uts; ++ut) o("V4 D", ut, " = {0, 0, 0, 0};");
            const std::string wcol = "(" + std::to_string(16 * wt) + " + row)";
            const bool wmask = 16 * wt + 15 >= p.mul_out;
            for (int k = 0; k < n3; ++k) {
                o("{");
                o.ind++;
                for (int m = 0; m < 4; ++m) {
                    if (wmask)
                        o("const T b", m, " = (bl", m, " && ", wcol, " < ", p.mul_out, ") ? g[(size_t)bn", m, " * DOUT + ", p.o, " + (",
                          wcol, " < ", p.mul_out, " ? ", wcol, " : 0) * ", n3, " + ", k, "] : (T)0;");
                    else
                        o("const T b", m, " = bl", m, " ? g[(size_t)bn", m, " * DOUT + ", p.o, " + ", wcol, " * ", n3, " + ", k,
                          "] : (T)0;");
                }
                for (int ut = 0; ut < uts; ++ut) {
                    const std::string u = "(" + std::to_string(16 * ut) + " + row)";
                    const bool umask = 16 * ut + 15 >= mp;
                    for (int m = 0; m < 4; ++m) {
                        const std::string base = std::to_string(loff[pi] + 16 * mp * k);
                        const std::string rr = "(" + std::to_string(4 * m) + " + usub)";
                        if (umask)
                            o("D", ut, " = MFMA(", u, " < ", mp, " ? lds[", base, " + TSW((", u, " < ", mp, " ? ", u, " : 0), ", rr,
                              ")] : (T)0, b", m, ", D", ut, ");");
                        else
                            o("D", ut, " = MFMA(lds[", base, " + TSW(", u, ", ", rr, ")], b", m, ", D", ut, ");");
                    }
                }
                o.ind--;
                o("}");
            }
            // lane holds D[u = 16 ut + U(v)][w = 16 wt + lane % 16]
            for (int ut = 0; ut < uts; ++ut)
                for (int v = 0; v < 4; ++v) {
                    const std::string uu = "(" + std::to_string(16 * ut) + " + " + uvb_u(f64, v) + ")";
                    std::string guard;
                    if (16 * ut + 15 >= p.mul_in) guard += uu + " < " + std::to_string(p.mul_in);
                    if (wmask) guard += (guard.empty() ? "" : " && ") + wcol + " < " + std::to_string(p.mul_out);
                    o(guard.empty() ? "" : "if (" + guard + ") ", "ws[(size_t)tile * WN + ", p.w_off, " + ", uu, " * ", p.mul_out, " + ", wcol,
                      "] = D", ut, "[", v, "];");
                }
            o.ind--;
            o("}");
        }
    }
    o.ind--;
    o("}");
    o("");
}

void emit_ucb_kernels(Out &o, const Plan &P)
{
    o("#define WN ", P.w_numel, "L");
    int dg = 0;
    for (const Path &p : P.paths) dg += p.mul_in * n_of(p.l3);
    o("#define DG ", dg);
    emit_ucb_g_kernel(o, P);
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi) emit_ucb_w_group(o, P, gi);
    o("// one workgroup of ", 16 / P.uvc_rpw, " waves per 16 receivers; `group` selects the path group");
    o("extern \"C\" __global__ void __launch_bounds__(", 1024 / P.uvc_rpw, ", ", P.uvc_waves_per_eu,
      ") cgtp_conv_uvw_bwd_w(const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, "
      "const T* __restrict__ y, const T* __restrict__ g, T* __restrict__ ws, long nrows, "
      "const int* __restrict__ order, int group)");
    o("{");
    o.ind++;
    o("__shared__ T lds[", uvc_lds_elems(P), "];  // T of the tile's 16 receivers, [p,k][u][row] (rows swizzled)");
    o("const long tile = blockIdx.x;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)P.uvc_groups.size(); ++gi)
        o("case ", gi, ": ucw_g", gi, "(tile, wv, lane, row_ptr, col, x, y, g, ws, nrows, order, lds); break;");
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
    emit_reduce_chunks(o);
}

}  // namespace

std::string generate_uvw_backward_source(const Plan &P)
{
    Out o;
    o("// @@section common");
    emit_preamble(o, P);
    emit_mfma_defs(o, P);
    o("// @@section cgtp_tp_uvw_bwd");
    emit_uvb_kernels(o, P);
    return o.s.str();
}

std::string generate_conv_uvw_backward_source(const Plan &P)
{
    Out o;
    o("// @@section common");
    emit_preamble(o, P);
    emit_mfma_defs(o, P);
    o("// @@section cgtp_conv_uvw_bwd");
    emit_ucb_kernels(o, P);
    o("// @@section cgtp_conv_uvw_acc");
    emit_uvc_acc_kernel(o, P);
    o("// @@section cgtp_conv_uvw_rad");
    emit_uvc_rad_kernel(o, P);
    return o.s.str();
}

int conv_uvw_g_items(const Plan &P, std::vector<std::pair<int, int>> *items) { return ucb_items(P, items); }

// receiver rows may be split over several waves only when one wave covers the whole receiver
bool fwd_splittable(const Plan &P) { return P.fwd_tasks == 1 && P.fwd_groups.size() == 1; }

int uvw_out_tiles(const Plan &P)
{
    int m = 1;
    for (const Irrep &o : P.out) m = std::max(m, o.mul);
    return (m + 15) / 16;
}

int fwd_group_accs(const Plan &P, int gi)
{
    int n = 0;
    for (int q : touched(P, P.fwd_groups[gi].paths).slots) n += n_of(P.out[q].l);
    return n;
}

int64_t conv_uvw_g_width(const Plan &P)
{
    int64_t dg = 0;
    for (const Path &p : P.paths) dg += (int64_t)p.mul_in * (2 * p.l3 + 1);
    return dg;
}

long radial_bwd_red_size(const Plan &P, int R, const std::vector<Group> &bwd_groups)
{
    long red = bwd_red_size(bwd_groups, P);
    for (const Group &g : bwd_groups) red = std::max<long>(red, 3L * std::min(kRadialRound, R * (int)g.paths.size()) * g.ct);
    return red;
}

// LDS words of the compact Theta copies (the largest unit of the launch)
long radial_fwd_theta_words(const Plan &P, int R)
{
    long m = 0;
    for (const Group &g : P.fwd_groups) m = std::max(m, (long)R * theta_width(P, g, true));
    return m;
}

long radial_bwd_theta_words(const Plan &P, int R, const std::vector<Group> &bwd_groups)
{
    long m = 0;
    for (const Group &g : bwd_groups) m = std::max(m, (long)R * theta_width(P, g, false));
    return m;
}

long radial_fwd_lds_bytes(const Plan &P, int R)
{
    return radial_fwd_theta_words(P, R) * (P.dtype == CGTP_F64 ? 8 : 4);
}

bool radial_fwd_fits(const Plan &P, int R) { return radial_fwd_lds_bytes(P, R) <= kLdsBytes; }

bool radial_bwd_fits(const Plan &P, int R, const std::vector<Group> &bwd_groups)
{
    return !bwd_groups.empty() &&
           (radial_bwd_theta_words(P, R, bwd_groups) + radial_bwd_red_size(P, R, bwd_groups)) *
                   (P.dtype == CGTP_F64 ? 8 : 4) <=
               kLdsBytes;
}

std::string generate_radial_source(const Plan &P, int R, const std::vector<Group> &bwd_groups, int bwd_waves)
{
    Out o;
    o("// @@section common");
    emit_preamble(o, P);
    o("#define NRAD ", R);
    o("#define WN ((long)NRAD * WROW)");
    emit_slot_sum(o, P);
    o("// @@section cgtp_conv_fwd_radial");
    if (!radial_fwd_fits(P, R)) {
        o("// forward not generated: the Theta columns of one path group's channel tile exceed the LDS");
    } else {
        for (int gi = 0; gi < (int)P.fwd_groups.size(); ++gi) emit_fwd_group(o, P, gi, false, false, R);
        o("// one wave per (receiver, path group, channel tile); the 4 waves of a workgroup share the");
        o("// (group, tile), whose Theta columns the workgroup first copies to LDS: block b takes unit");
        o("// b % units of receivers 4 (b / units) .. 4 (b / units) + 3, so a receiver's units run side by side");
        // the rebuilt weights and the double-buffered radial features need more registers than the
        // forward's target leaves (measured: spills at 4 waves per SIMD)
        const int waves = std::max(1, P.fwd_waves_per_eu - 1 - (R > 8 ? 1 : 0));
        o("extern \"C\" __global__ void __launch_bounds__(256, ", waves, ") cgtp_conv_fwd_radial("
          "const int* __restrict__ row_ptr, const int* __restrict__ col, const T* __restrict__ x, const T* __restrict__ y, "
          "const T* __restrict__ rho, const T* __restrict__ theta, T* __restrict__ out, long nrows, long nwaves, "
          "const int* __restrict__ order)");
        o("{");
        o.ind++;
        o("__shared__ T thl[", radial_fwd_theta_words(P, R), "];  // Theta columns of the unit, [r][col]");
        o("const int task = (int)(blockIdx.x % ", P.fwd_tasks, ");");
        o("const int lane = threadIdx.x & 63;");
        o("long n = (long)(blockIdx.x / ", P.fwd_tasks, ") * 4 + WAVE_IN_BLOCK();");
        o("const bool live = n < nrows;");
        o("if (live && order) n = order[n];  // receiver schedule (heavy rows first), results unchanged");
        o("const int part = 0;");
        o("T* pred = nullptr;");
        o("switch (task) {");
        int task = 0;
        const std::string targ = fwd_splittable(P) ? "<1>" : "";
        for (int gi = 0; gi < (int)P.fwd_groups.size(); ++gi)
            for (int tile = 0; tile < P.fwd_groups[gi].tiles; ++tile, ++task) {
                o("case ", task, ": {");
                o.ind++;
                o("const int tile = ", tile, ";");
                emit_theta_stage(o, P, P.fwd_groups[gi], R, true, "256");
                o("__syncthreads();");
                o("if (live) rad_g", gi, targ, "(n, tile, lane, row_ptr, col, x, y, rho, thl, out, nrows, part, live, pred);");
                o("break;");
                o.ind--;
                o("}");
            }
        o("default: break;");
        o("}");
        o.ind--;
        o("}");
        o("");
    }
    // backward: the sender pass with W rebuilt from rho and Theta and dW consumed into drho and
    // the chunk's dTheta partial (Sobek page, Abstract: no edge-sized weights or adjoints)
    o("// @@section cgtp_conv_bwd_radial");
    const long red = radial_bwd_red_size(P, R, bwd_groups);
    if (!radial_bwd_fits(P, R, bwd_groups)) {
        o("// backward not generated: a path group's Theta columns and the reduction buffer exceed the LDS");
        return o.s.str();
    }
    for (int gi = 0; gi < (int)bwd_groups.size(); ++gi) emit_bwd_group(o, P, gi, false, false, R, &bwd_groups);
    o("// one workgroup of 64*wpr threads per chunk of spc consecutive senders; `group` selects the path group,");
    o("// whose Theta columns the workgroup first copies to LDS");
    o("extern \"C\" __global__ void __launch_bounds__(256, ", bwd_waves, ") cgtp_conv_bwd_radial("
      "const int* __restrict__ t_row_ptr, const int* __restrict__ t_edge, const int* __restrict__ t_dst, "
      "const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ rho, const T* __restrict__ theta, "
      "const T* __restrict__ g, T* __restrict__ dx, T* __restrict__ dy, T* __restrict__ drho, T* __restrict__ ws, "
      "long nnodes, long spc, int wpr, int group)");
    o("{");
    o.ind++;
    o("__shared__ T thl[", radial_bwd_theta_words(P, R, bwd_groups), "];  // Theta columns of the group, [r][col]");
    o("__shared__ T red[", red, "];  // partial dx / dTheta of waves 1..3");
    // an opaque zero offset keeps the compiler from hoisting every Theta read out of the edge loop
    o("int zo = 0;");
    o("asm volatile(\"\" : \"+v\"(zo));");
    o("const T* th = thl + zo;");
    o("const long chunk = blockIdx.x;");
    o("const long c0 = chunk * spc;");
    o("const long c1 = c0 + spc < nnodes ? c0 + spc : nnodes;");
    o("const int wv = WAVE_IN_BLOCK();");
    o("const int lane = threadIdx.x & 63;");
    o("switch (group) {");
    for (int gi = 0; gi < (int)bwd_groups.size(); ++gi) {
        o("case ", gi, ": {");
        o.ind++;
        emit_theta_stage(o, P, bwd_groups[gi], R, false, "blockDim.x");
        o("__syncthreads();");
        o("rbw_g", gi, "(chunk, c0, c1, wv, lane, wpr, red, t_row_ptr, t_edge, t_dst, x, y, rho, th, g, dx, dy, drho, ws);");
        o("break;");
        o.ind--;
        o("}");
    }
    o("default: break;");
    o("}");
    o.ind--;
    o("}");
    o("");
    emit_reduce_chunks(o);
    return o.s.str();
}

std::string generate_source(const Plan &P)
{
    // "// @@section NAME" lines split the module into the shared preamble and one part per
    // kernel (with its helpers), so a measurement taken on one kernel can be matched to the
    // exact code it ran even after other kernels of the module change.
    Out o;
    o("// @@section common");
    emit_preamble(o, P);
    if (P.unit_weights) {
        // internal plan of the uvw convolution backward: the sender pass only
        emit_slot_sum(o, P);
        o("// @@section cgtp_conv_uvw_bwd_xy");
        emit_bwd_kernel(o, P);
    } else if (P.mode == CGTP_UVU) {
        emit_slot_sum(o, P);
        o("// @@section cgtp_conv_fwd");
        for (int gi = 0; gi < (int)P.fwd_groups.size(); ++gi) emit_fwd_group(o, P, gi, false);
        emit_fwd_kernel(o, P, false);
        // the same pass with each receiver row split over 2 or 4 waves (a `_splitN` section
        // holds only the entry point; its code is the base section's template)
        if (fwd_splittable(P))
            for (int split : {2, 4}) {
                o("// @@section cgtp_conv_fwd", split_suffix(split));
                emit_fwd_kernel(o, P, false, false, split);
            }
        o("// @@section cgtp_tp_fwd");
        for (int gi = 0; gi < (int)P.fwd_groups.size(); ++gi) emit_fwd_group(o, P, gi, true);
        emit_fwd_kernel(o, P, true);
        o("// @@section cgtp_conv_bwd");
        emit_bwd_kernel(o, P);
        o("// @@section cgtp_conv_rbw");
        emit_rbw_kernels(o, P);
        o("// @@section cgtp_tp_bwd");
        emit_tpb_kernel(o, P);
        o("// @@section cgtp_conv_dbwd_recv");
        for (int gi = 0; gi < (int)P.fwd_groups.size(); ++gi) emit_fwd_group(o, P, gi, false, true);
        emit_fwd_kernel(o, P, false, true);
        if (fwd_splittable(P))
            for (int split : {2, 4}) {
                o("// @@section cgtp_conv_dbwd_recv", split_suffix(split));
                emit_fwd_kernel(o, P, false, true, split);
            }
        o("// @@section cgtp_conv_dbwd_send");
        emit_bwd_kernel(o, P, true);
    } else {
        emit_mfma_defs(o, P);
        o("// @@section cgtp_tp_uvw");
        emit_uvw_kernel(o, P);
        o("// @@section cgtp_conv_uvw");
        emit_uvc_kernel(o, P);
    }
    return o.s.str();
}

}  // namespace cgtp
