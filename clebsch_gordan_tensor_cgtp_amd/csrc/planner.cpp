// Host planner of libcgtp: irreps grammar, coupling paths, output slots, the
// real CG blocks and the work split of the generated kernels.
//
// The CG values are computed here with the lowering-operator recursion (the
// highest-weight state fixed by J+|J J> = 0, then J- applied M times), in long
// double.  This is deliberately a different algorithm from a closed-form
// Racah sum so that the two independent codes cross-check each other.  The
// real basis, the Frobenius-1 normalisation, the sign rule and the zero
// threshold are the conventions stated in include/cgtp.h.
//
// Pages: sciencestack.ai page (TL;DR, Abstract, Figures 1-3): static analysis
// of the block-sparse CG tensor at model compile time, blocks that are
// themselves sparse and repeated; "The GPU memory optimization with Larger
// angular momentum" discussion: nonzeros coded into the instruction stream.
#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdlib>
#include <complex>
#include <map>
#include <set>
#include <sstream>

#include "plan.h"

namespace cgtp {

static constexpr int kLmax = 7;
static constexpr long double kZeroTol = 1e-9L;

std::vector<Irrep> parse_irreps(const std::string &text, const char *what)
{
    std::string s;
    for (char ch : text)
        if (!std::isspace(static_cast<unsigned char>(ch))) s.push_back(ch);
    if (s.empty()) throw Error(CGTP_ERR_IRREPS, std::string(what) + " irreps: empty string");
    std::vector<Irrep> out;
    size_t pos = 0;
    while (pos <= s.size()) {
        size_t plus = s.find('+', pos);
        std::string term = s.substr(pos, plus == std::string::npos ? std::string::npos : plus - pos);
        auto bad = [&](const char *why) {
            return Error(CGTP_ERR_IRREPS, std::string(what) + " irreps: term '" + term + "' " + why);
        };
        size_t x = term.find('x');
        if (x == std::string::npos || x == 0) throw bad("must look like MULxLP");
        for (size_t i = 0; i < x; ++i)
            if (!std::isdigit(static_cast<unsigned char>(term[i]))) throw bad("has a bad multiplicity");
        if (term.size() < x + 3) throw bad("lacks L or parity");
        char par = term.back();
        if (par != 'e' && par != 'o') throw bad("parity must be e or o");
        std::string lstr = term.substr(x + 1, term.size() - x - 2);
        for (char ch : lstr)
            if (!std::isdigit(static_cast<unsigned char>(ch))) throw bad("has a bad L");
        if (x > 9 || lstr.size() > 3) throw bad("is out of range");
        Irrep ir;
        ir.mul = std::stoi(term.substr(0, x));
        ir.l = std::stoi(lstr);
        ir.p = par == 'e' ? 1 : -1;
        if (ir.mul < 1) throw bad("needs multiplicity >= 1");
        if (ir.l > kLmax) throw bad("has L above 7");
        out.push_back(ir);
        if (plus == std::string::npos) break;
        pos = plus + 1;
    }
    return out;
}

// ------------------------------------------------------------------------------------------
// Complex CG by recursion.  table[m1 + j1][M + J] holds <j1 m1, j2 M-m1 | J M>.

static long double raise_coef(int j, int m) { return std::sqrt((long double)(j - m) * (j + m + 1)); }
static long double lower_coef(int j, int m) { return std::sqrt((long double)(j + m) * (j - m + 1)); }

static std::vector<std::vector<long double>> complex_cg_table(int j1, int j2, int J)
{
    std::vector<std::vector<long double>> t(2 * j1 + 1, std::vector<long double>(2 * J + 1, 0.0L));
    auto at = [&](int m1, int M) -> long double & { return t[m1 + j1][M + J]; };
    auto valid = [&](int m1, int M) { return std::abs(m1) <= j1 && std::abs(M - m1) <= j2 && std::abs(M) <= J; };
    // highest weight M = J: J+ |J J> = 0 gives
    //   a(m1+1) raise_coef(j2, J-m1-1) + a(m1) raise_coef(j1, m1) = 0
    // with a(j1) > 0 (Condon-Shortley).
    int lo = std::max(-j1, J - j2);
    at(j1, J) = 1.0L;
    for (int m1 = j1 - 1; m1 >= lo; --m1) at(m1, J) = -at(m1 + 1, J) * raise_coef(j2, J - m1 - 1) / raise_coef(j1, m1);
    long double nrm = 0.0L;
    for (int m1 = lo; m1 <= j1; ++m1) nrm += at(m1, J) * at(m1, J);
    nrm = std::sqrt(nrm);
    for (int m1 = lo; m1 <= j1; ++m1) at(m1, J) /= nrm;
    // lowering: lower_coef(J, M) |J M-1> = (J1- + J2-) |J M>
    for (int M = J; M > -J; --M) {
        for (int m1 = -j1; m1 <= j1; ++m1) {
            int m2 = M - 1 - m1;
            if (!valid(m1, M - 1)) continue;
            long double v = 0.0L;
            if (m1 + 1 <= j1 && valid(m1 + 1, M)) v += at(m1 + 1, M) * lower_coef(j1, m1 + 1);
            if (m2 + 1 <= j2 && valid(m1, M)) v += at(m1, M) * lower_coef(j2, m2 + 1);
            at(m1, M - 1) = v / lower_coef(J, M);
        }
    }
    return t;
}

// Row r = m + l of the real-basis matrix Q_l (real = Q complex): up to two entries.
struct QEntry {
    int m;
    std::complex<long double> v;
};
static std::vector<QEntry> q_row(int l, int m)
{
    const long double s = 1.0L / std::sqrt(2.0L);
    const long double sg = (m % 2 == 0) ? 1.0L : -1.0L;
    if (m > 0) return {{-m, {s, 0}}, {m, {sg * s, 0}}};
    if (m < 0) return {{m, {0, s}}, {-m, {0, -sg * s}}};
    return {{0, {1, 0}}};
}

std::vector<Nonzero> real_cg_nonzeros(int l1, int l2, int l3)
{
    if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) throw Error(CGTP_ERR_INTERNAL, "triangle rule");
    auto cg = complex_cg_table(l1, l2, l3);
    const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
    std::vector<long double> part(n1 * n2 * n3, 0.0L);
    const bool take_real = (l1 + l2 + l3) % 2 == 0;
    for (int i = 0; i < n1; ++i)
        for (int j = 0; j < n2; ++j)
            for (int k = 0; k < n3; ++k) {
                std::complex<long double> acc = 0;
                for (const auto &a : q_row(l1, i - l1))
                    for (const auto &b : q_row(l2, j - l2))
                        for (const auto &c : q_row(l3, k - l3)) {
                            if (a.m + b.m != c.m) continue;
                            acc += std::conj(a.v) * std::conj(b.v) * c.v * cg[a.m + l1][c.m + l3];
                        }
                part[(i * n2 + j) * n3 + k] = take_real ? acc.real() : acc.imag();
            }
    long double nrm = 0.0L;
    for (long double v : part) nrm += v * v;
    nrm = std::sqrt(nrm);
    long double sign = 0.0L;
    for (long double &v : part) {
        v /= nrm;
        if (std::fabs(v) <= kZeroTol) v = 0.0L;
        if (sign == 0.0L && v != 0.0L) sign = v > 0 ? 1.0L : -1.0L;
    }
    std::vector<Nonzero> nz;
    for (int i = 0; i < n1; ++i)
        for (int j = 0; j < n2; ++j)
            for (int k = 0; k < n3; ++k) {
                long double v = part[(i * n2 + j) * n3 + k];
                if (v != 0.0L) nz.push_back({i, j, k, static_cast<double>(sign * v)});
            }
    return nz;
}

// ------------------------------------------------------------------------------------------

void build_paths(Plan &P)
{
    for (const Irrep &s : P.sh)
        if (s.mul != 1) throw Error(CGTP_ERR_IRREPS, "every SH irrep must have multiplicity 1");
    std::vector<int> xo, yo, oo;
    int acc = 0;
    for (const Irrep &r : P.ins) { xo.push_back(acc); acc += r.dim(); }
    P.d_x = acc;
    acc = 0;
    for (const Irrep &r : P.sh) { yo.push_back(acc); acc += r.dim(); }
    P.d_sh = acc;
    acc = 0;
    for (const Irrep &r : P.out) { oo.push_back(acc); acc += r.dim(); }
    P.d_out = acc;

    auto in_out = [&](int l, int p) {
        for (const Irrep &o : P.out)
            if (o.l == l && o.p == p) return true;
        return false;
    };
    std::vector<Path> paths;
    for (int i1 = 0; i1 < (int)P.ins.size(); ++i1)
        for (int i2 = 0; i2 < (int)P.sh.size(); ++i2) {
            const Irrep &a = P.ins[i1], &b = P.sh[i2];
            for (int l3 = std::abs(a.l - b.l); l3 <= a.l + b.l; ++l3) {
                int p3 = a.p * b.p;
                if (!in_out(l3, p3)) continue;
                Path p{};
                p.i1 = i1; p.i2 = i2; p.l1 = a.l; p.l2 = b.l; p.l3 = l3; p.p3 = p3;
                p.a = xo[i1]; p.b = yo[i2];
                p.slot = -1;
                paths.push_back(p);
            }
        }
    // output slots: key (l, p) -> occurrences in out, producing paths in order
    std::map<std::pair<int, int>, std::vector<int>> occ, prod;
    for (int q = 0; q < (int)P.out.size(); ++q) occ[{P.out[q].l, P.out[q].p}].push_back(q);
    for (int i = 0; i < (int)paths.size(); ++i) prod[{paths[i].l3, paths[i].p3}].push_back(i);
    for (auto &kv : occ) {
        auto it = prod.find(kv.first);
        std::ostringstream key;
        key << "l=" << kv.first.first << (kv.first.second > 0 ? "e" : "o");
        if (it == prod.end()) throw Error(CGTP_ERR_IRREPS, "output irrep " + key.str() + " is produced by no path");
        const auto &pr = it->second;
        if (kv.second.size() == 1) {
            for (int i : pr) paths[i].slot = kv.second[0];
        } else if (kv.second.size() == pr.size()) {
            for (size_t t = 0; t < pr.size(); ++t) paths[pr[t]].slot = kv.second[t];
        } else {
            std::ostringstream m;
            m << "output irrep " << key.str() << " occurs " << kv.second.size() << " times but " << pr.size()
              << " paths produce it";
            throw Error(CGTP_ERR_IRREPS, m.str());
        }
    }
    int64_t w = 0;
    P.nnz_total = 0;
    std::map<std::tuple<int, int, int>, std::vector<Nonzero>> cache;
    for (Path &p : paths) {
        p.o = oo[p.slot];
        p.mul_in = P.ins[p.i1].mul;
        p.mul_out = P.out[p.slot].mul;
        if (P.mode == CGTP_UVU && p.mul_out != p.mul_in)
            throw Error(CGTP_ERR_IRREPS, "uvu needs the output multiplicity to equal the input's on every path");
        p.w_off = w;
        w += P.mode == CGTP_UVU ? p.mul_in : (int64_t)p.mul_in * p.mul_out;
        auto key = std::make_tuple(p.l1, p.l2, p.l3);
        auto c = cache.find(key);
        if (c == cache.end()) c = cache.emplace(key, real_cg_nonzeros(p.l1, p.l2, p.l3)).first;
        p.nz = c->second;
        P.nnz_total += (int)p.nz.size();
    }
    if (paths.empty()) throw Error(CGTP_ERR_IRREPS, "no coupling path connects the irreps");
    P.w_numel = w;
    P.paths = std::move(paths);
}

// ------------------------------------------------------------------------------------------
// Work split.  Forward: output slots are grouped by the input blocks their
// paths read (path-group parallelism, LunaTP page, Abstract), so each x
// block is read by one group only; a class whose accumulators exceed the
// register budget is split.  Each (receiver, group, channel tile) is one
// wave.  Backward: one group with every path (the sender pass keeps only the
// input gradient resident, so it needs no path split and each edge's dY is
// complete inside one wave).

static int lanes_for(int mul)
{
    int ct = 1;
    while (ct < mul && ct < 64) ct *= 2;
    return ct;
}

static void finish_group(Group &g)
{
    g.ct = lanes_for(g.mul);
    g.es = 64 / g.ct;
    g.tiles = (g.mul + g.ct - 1) / g.ct;
}

static int getenv_int(const char *name, int dflt)
{
    const char *e = std::getenv(name);
    return e && *e ? std::max(1, std::atoi(e)) : dflt;
}

// 32-bit registers per lane of one sender-pass group: dx accumulators and x per sender, the edge
// operands (y, W, g), dY partials, the B block and its contractions; the double backward adds
// ggx, ggy, ggw and a second contraction per line; the radial backward (R features) replaces W
// by the R radial features and adds R dTheta sums per path and R drho partials.
static int sender_estimate(const Plan &P, const std::vector<int> &ps, bool prefetch, bool dbl, int radial)
{
    const int word = P.dtype == CGTP_F64 ? 2 : 1;
    std::set<int> i1s, i2s, slots;
    int maxb = 0;
    for (int pi : ps) {
        std::set<std::pair<int, int>> ij;
        for (const Nonzero &z : P.paths[pi].nz) ij.insert({z.i, z.j});
        i1s.insert(P.paths[pi].i1);
        i2s.insert(P.paths[pi].i2);
        slots.insert(P.paths[pi].slot);
        maxb = std::max(maxb, (int)ij.size() + (dbl ? 2 : 1) * (2 * P.paths[pi].l1 + 2 * P.paths[pi].l2 + 2));
    }
    int xs = 0, ys = 0, gs = 0;
    for (int b : i1s) xs += 2 * P.ins[b].l + 1;
    for (int b : i2s) ys += 2 * P.sh[b].l + 1;
    for (int q : slots) gs += 2 * P.out[q].l + 1;
    const int wregs = radial ? radial : (int)ps.size();
    int edge = ys + wregs + gs + (dbl ? ys + (int)ps.size() : 0);
    const int extra = radial ? radial * ((int)ps.size() + 1) : 0;
    return word * ((dbl ? 3 : 2) * xs + edge + ys + maxb + extra + (prefetch ? edge : 0)) + 24;
}

// Radial-projection backward (R features): sender-pass groups packed per SH block while the
// estimate fits the budget (a group holds at least one path); occupancy target from the largest.
std::vector<Group> radial_bwd_groups(const Plan &P, int R, int &waves)
{
    // measured on the NequIP-like graph: 220 registers (fewer launches at 2 waves per SIMD) is best
    // up to R = 8 (R = 8: 458 us against 570 us at 168), 168 above (R = 16: 797 us against 1185 us)
    const int budget = getenv_int("CGTP_RAD_BUDGET", R <= 8 ? 220 : 168);
    std::vector<Group> groups;
    std::vector<int> all;
    for (int i = 0; i < (int)P.paths.size(); ++i) all.push_back(i);
    if (sender_estimate(P, all, false, false, R) <= budget) {
        Group g;
        g.paths = all;
        groups.push_back(g);
    } else {
        for (int b = 0; b < (int)P.sh.size(); ++b) {
            Group cur;
            for (int i = 0; i < (int)P.paths.size(); ++i) {
                if (P.paths[i].i2 != b) continue;
                std::vector<int> trial = cur.paths;
                trial.push_back(i);
                if (!cur.paths.empty() && sender_estimate(P, trial, false, false, R) > budget) {
                    groups.push_back(cur);
                    cur = Group();
                }
                cur.paths.push_back(i);
            }
            if (!cur.paths.empty()) groups.push_back(cur);
        }
    }
    int est_max = 0;
    for (Group &g : groups) {
        for (int pi : g.paths) g.mul = std::max(g.mul, P.paths[pi].mul_in);
        finish_group(g);
        g.prefetch = false;
        est_max = std::max(est_max, sender_estimate(P, g.paths, false, false, R));
    }
    waves = std::max(1, std::min(4, 512 * 4 / (5 * std::max(est_max, 1))));
    waves = getenv_int("CGTP_RAD_WAVES", waves);
    return groups;
}

void schedule(Plan &P)
{
    if (const char *e = std::getenv("CGTP_BWD_PREFETCH")) P.bwd_prefetch = std::atoi(e);
    if (const char *e = std::getenv("CGTP_FWD_SPLIT_INPUTS")) P.fwd_split_inputs = std::atoi(e) != 0;
    if (const char *e = std::getenv("CGTP_NT")) P.stream_hint = std::atoi(e) != 0;
    if (const char *e = std::getenv("CGTP_SCALAR_WAVE")) P.scalar_wave = std::atoi(e) != 0;
    const int word = P.dtype == CGTP_F64 ? 2 : 1;
    // 32-bit registers per lane for the forward accumulators (CGTP_FWD_BUDGET overrides, tuning).
    // An fp64 plan that needs more than two groups at 64 registers already runs at two waves per
    // SIMD, which leaves room for twice that budget: on the MACE-like plan 3 path groups instead of
    // 5 (fewer re-reads of the sender row), 232 VGPRs and no spill, 12.08 -> 10.6 ms.  A smaller
    // plan keeps 64: the NequIP-like fp64 plan in one group needs 208 VGPRs (two waves per SIMD,
    // 362 us) against two groups at 122 (four waves, 296 us).  fp32 with 128 at two waves on the
    // MACE-like plan: 5.20 against 4.63 ms.
    int total_need = 0;
    if (P.mode == CGTP_UVU)
        for (const Irrep &o : P.out) total_need += word * (2 * o.l + 1);
    const int budget =
        std::max(16, getenv_int("CGTP_FWD_BUDGET", word == 2 && total_need > 2 * 64 ? 128 : 64));
    // Receiver-order backward: the same grouping with a smaller budget for the gradient values
    // each lane holds (besides them it keeps the edge's operands, its dx contribution and dY
    // partials live), so that a group stays near 128 registers.
    // Measured (MI355X, receiver-order backward): a plan whose gradient row fits 64 registers runs
    // fastest in one group (10M-edge graph 30.8 ms against 36.3 at 32); larger plans at 32 (the
    // MACE-like plan: 24.5 ms against 28.1 at 64, fp64 68.8 against 117).
    const int rbw_budget = std::max(8, getenv_int("CGTP_RBW_BUDGET", total_need <= 64 ? 64 : 32));
    auto make_slot_groups = [&](int budget, std::vector<Group> &groups) {
    groups.clear();
    if (P.mode == CGTP_UVU) {
        std::vector<std::vector<int>> slot_paths(P.out.size());
        for (int i = 0; i < (int)P.paths.size(); ++i) slot_paths[P.paths[i].slot].push_back(i);
        auto inputs_of = [&](int q) {
            std::vector<int> v;
            for (int i : slot_paths[q]) v.push_back(P.paths[i].i1);
            std::sort(v.begin(), v.end());
            v.erase(std::unique(v.begin(), v.end()), v.end());
            return v;
        };
        // slots in order of their first path, so input blocks stay together
        std::vector<int> order;
        for (int q = 0; q < (int)P.out.size(); ++q) order.push_back(q);
        std::stable_sort(order.begin(), order.end(),
                         [&](int a, int b) { return slot_paths[a].front() < slot_paths[b].front(); });
        Group cur;
        std::vector<int> cur_inputs;
        int regs = 0;
        auto need_of = [&](int q) { return word * (2 * P.out[q].l + 1); };
        int total = 0;
        for (int q : order) total += need_of(q);
        // A plan that needs several groups anyway keeps each input class (consecutive slots
        // fed by the same input blocks) whole where it fits: every group then gathers only
        // its own blocks of the sender row instead of re-reading blocks that the previous
        // group read too.
        bool pack = total > budget && !P.fwd_split_inputs;
        if (const char *e = std::getenv("CGTP_FWD_PACK_INPUTS")) pack = pack && std::atoi(e) != 0;
        std::vector<int> class_need(order.size(), 0);  // need of the class starting at position k
        for (int k = 0; k < (int)order.size();) {
            int j = k, sum = 0;
            while (j < (int)order.size() && inputs_of(order[j]) == inputs_of(order[k]) &&
                   P.out[order[j]].mul == P.out[order[k]].mul)
                sum += need_of(order[j++]);
            class_need[k] = sum;
            k = j;
        }
        for (int k = 0; k < (int)order.size(); ++k) {
            const int q = order[k];
            int need = need_of(q);
            int mul = P.out[q].mul;
            std::vector<int> ins = inputs_of(q);
            const bool class_start = class_need[k] > 0;
            const bool keep_class = pack && class_start && class_need[k] <= budget && regs + class_need[k] > budget;
            if (!cur.paths.empty() && (regs + need > budget || mul != cur.mul || keep_class ||
                                       (P.fwd_split_inputs && ins != cur_inputs))) {
                finish_group(cur);
                groups.push_back(cur);
                cur = Group();
                regs = 0;
            }
            cur.mul = mul;
            cur_inputs = ins;
            for (int i : slot_paths[q]) cur.paths.push_back(i);
            regs += need;
        }
        if (!cur.paths.empty()) {
            finish_group(cur);
            groups.push_back(cur);
        }
        for (Group &g : groups) std::sort(g.paths.begin(), g.paths.end());
    }
    };
    make_slot_groups(budget, P.fwd_groups);
    make_slot_groups(rbw_budget, P.rbw_groups);
    P.fwd_tasks = 0;
    for (const Group &g : P.fwd_groups) P.fwd_tasks += g.tiles;

    // uvw: output slots in order, packed while the MFMA accumulators (4 per lane
    // per output component) fit 64 registers; all paths of a slot stay together.
    P.uvw_groups.clear();
    if (P.mode == CGTP_UVW) {
        std::vector<std::vector<int>> slot_paths(P.out.size());
        for (int i = 0; i < (int)P.paths.size(); ++i) slot_paths[P.paths[i].slot].push_back(i);
        Group cur;
        int regs = 0;
        for (int q = 0; q < (int)P.out.size(); ++q) {
            if (slot_paths[q].empty()) continue;
            int need = 4 * word * (2 * P.out[q].l + 1);
            if (!cur.paths.empty() && regs + need > 64) {
                P.uvw_groups.push_back(cur);
                cur = Group();
                regs = 0;
            }
            for (int i : slot_paths[q]) cur.paths.push_back(i);
            regs += need;
        }
        if (!cur.paths.empty()) P.uvw_groups.push_back(cur);
        for (Group &g : P.uvw_groups) {
            std::sort(g.paths.begin(), g.paths.end());
            for (int pi : g.paths) g.mul = std::max(g.mul, P.paths[pi].mul_in);
        }
    }

    // uvw convolution: paths in slot order, packed while the per-lane sums T_p
    // (2l3+1 per path) fit 64 registers and the workgroup's staging of T for 16
    // receivers (16 * mul_in rounded to 4 * (2l3+1) per path) fits the LDS budget.
    // Workgroup shape: one receiver per wave (16 waves, 4 per SIMD, <= 128 VGPRs)
    // when the per-lane estimate fits, else 2 or 4 receivers per wave.  A 16-wave
    // workgroup fills a CU alone, so it may stage up to 120 KB; smaller ones keep
    // 64 KB so that two fit.
    P.uvc_groups.clear();
    if (P.mode == CGTP_UVW) {
        auto make = [&](long lds_budget, std::vector<Group> &groups) {
            groups.clear();
            std::vector<int> order;
            for (int q = 0; q < (int)P.out.size(); ++q)
                for (int i = 0; i < (int)P.paths.size(); ++i)
                    if (P.paths[i].slot == q) order.push_back(i);
            Group cur;
            int regs = 0;
            long lds = 0;
            for (int i : order) {
                const Path &p = P.paths[i];
                int need = word * (2 * p.l3 + 1);
                long bytes = 16L * ((p.mul_in + 3) / 4 * 4) * (2 * p.l3 + 1) * 4 * word;
                if (!cur.paths.empty() && (regs + need > 64 || lds + bytes > lds_budget)) {
                    groups.push_back(cur);
                    cur = Group();
                    regs = 0;
                    lds = 0;
                }
                cur.paths.push_back(i);
                regs += need;
                lds += bytes;
            }
            if (!cur.paths.empty()) groups.push_back(cur);
            int est_max = 0;
            for (Group &g : groups) {
                for (int pi : g.paths) g.mul = std::max(g.mul, P.paths[pi].mul_in);
                finish_group(g);
                std::set<int> i1s, i2s;
                int acc = 0;
                for (int pi : g.paths) {
                    i1s.insert(P.paths[pi].i1);
                    i2s.insert(P.paths[pi].i2);
                    acc += 2 * P.paths[pi].l3 + 1;
                }
                int ops = 0;
                for (int b : i1s) ops += 2 * P.ins[b].l + 1;
                for (int b : i2s) ops += 2 * P.sh[b].l + 1;
                // x_i * y_j products of the largest (input block, SH block) pair, live together
                std::map<std::pair<int, int>, std::set<std::pair<int, int>>> pair_ij;
                for (int pi : g.paths)
                    for (const Nonzero &z : P.paths[pi].nz) pair_ij[{P.paths[pi].i1, P.paths[pi].i2}].insert({z.i, z.j});
                int maxpair = 0;
                for (auto &kv : pair_ij) maxpair = std::max(maxpair, (int)kv.second.size());
                // fp64: register pairs and 64-bit address arithmetic measured ~30% above the count
                est_max = std::max(est_max, (word * (acc + 3 * ops / 2 + maxpair) + 24) * (word == 2 ? 13 : 10) / 10);
            }
            return est_max <= 128 ? 1 : est_max <= 256 ? 2 : 4;
        };
        P.uvc_rpw = make(65536, P.uvc_groups);
        const char *wide_env = std::getenv("CGTP_UVC_WIDE");
        if (P.uvc_rpw == 1 && (!wide_env || std::atoi(wide_env) != 0)) {
            std::vector<Group> wide;
            if (make(122880, wide) == 1) P.uvc_groups = wide;
        }
        // A group is split only between paths, so one path whose staging alone exceeds the
        // workgroup's LDS (e.g. 128x7o in fp64) cannot run: such plans keep the batched product
        // but the convolution kernels are not generated and their entry points report it.
        const long lds_cap = 160L * 1024;  // LDS of one gfx950 workgroup
        P.uvc_ok = true;
        for (const Group &g : P.uvc_groups) {
            long bytes = 0;
            for (int pi : g.paths) {
                const Path &p = P.paths[pi];
                bytes += 16L * ((p.mul_in + 3) / 4 * 4) * (2 * p.l3 + 1) * 4 * word;
            }
            if (bytes > lds_cap && P.uvc_ok) {
                P.uvc_ok = false;
                P.uvc_why = "uvw convolution: path " + std::to_string(g.paths.front()) + " stages " +
                            std::to_string(bytes) + " bytes of T for a 16-receiver tile, more than the " +
                            std::to_string(lds_cap) + " bytes of LDS of one workgroup";
            }
        }
        if (!P.uvc_ok) P.uvc_groups.clear();
    }

    // uvw batched backward: dx/dy groups are the input blocks (each block's dx is complete in one
    // launch; dY is accumulated over the launches in order); dW groups pack 8 paths (a 16x16
    // MFMA accumulator, 4 registers per lane, per path; 16 spilled at l = 7).
    P.uvb_x_groups.clear();
    P.uvb_w_groups.clear();
    P.uvb_ok = P.mode == CGTP_UVW;
    if (P.mode == CGTP_UVW) {
        for (const Path &p : P.paths) P.uvb_ok = P.uvb_ok && p.mul_in <= 16 && p.mul_out <= 16;
        for (int b = 0; b < (int)P.ins.size(); ++b) {
            Group g;
            for (int i = 0; i < (int)P.paths.size(); ++i)
                if (P.paths[i].i1 == b) g.paths.push_back(i);
            if (!g.paths.empty()) P.uvb_x_groups.push_back(g);
        }
        // The kernel's four waves per 16-row block take the input blocks by cost; a block heavier
        // than an eighth of the whole is split into two path halves of about equal cost, which
        // two waves run (each adds its dx partial in LDS, summed in fixed order at the end), so
        // that no wave carries much more than a quarter.
        if (getenv_int("CGTP_UVB_XY_SPLIT", 1)) {
            auto cost = [&](int pi) {
                const Path &p = P.paths[pi];
                return (long)p.nz.size() * 6 + 16L * (2 * p.l3 + 1);
            };
            long total = 0;
            for (const Group &g : P.uvb_x_groups)
                for (int pi : g.paths) total += cost(pi);
            std::vector<Group> out;
            for (const Group &g : P.uvb_x_groups) {
                long c = 0;
                for (int pi : g.paths) c += cost(pi);
                if (g.paths.size() < 2 || 8 * c <= total) {
                    out.push_back(g);
                    continue;
                }
                Group h1, h2;
                h1.part = 1;
                h2.part = 2;
                long acc = 0;
                for (int pi : g.paths) {
                    if (2 * (acc + cost(pi)) <= c || h1.paths.empty())
                        h1.paths.push_back(pi), acc += cost(pi);
                    else
                        h2.paths.push_back(pi);
                }
                if (h2.paths.empty()) {
                    out.push_back(g);
                    continue;
                }
                out.push_back(h1);
                out.push_back(h2);
            }
            // the halves' dx partials live in LDS next to the dY rows: 16 x (16 (2 l1 + 1) + 1)
            // words per half, within the 160 KB of a workgroup (the fp64 l <= 7 plan does not fit
            // and keeps its blocks whole)
            long words = 4L * 16 * (P.d_sh | 1);
            for (const Group &g : out)
                if (g.part) words += 16L * (16 * (2 * P.ins[P.paths[g.paths[0]].i1].l + 1) + 1);
            if (words * (P.dtype == CGTP_F64 ? 8 : 4) <= 160L * 1024) P.uvb_x_groups = out;
        }
        Group cur;
        for (int i = 0; i < (int)P.paths.size(); ++i) {
            if ((int)cur.paths.size() == (getenv_int("CGTP_UVB_W_PATHS", 8))) {
                P.uvb_w_groups.push_back(cur);
                cur = Group();
            }
            cur.paths.push_back(i);
        }
        if (!cur.paths.empty()) P.uvb_w_groups.push_back(cur);
    }

    // Sender-pass groups (backward, and the double backward's d/dx, d/dy, d/dW):
    // paths sharing an SH block (so that block's dY is complete in one group),
    // split when the register estimate exceeds the budget.
    {
        auto estimate = [&](const std::vector<int> &ps, bool prefetch, bool dbl) {
            return sender_estimate(P, ps, prefetch, dbl, 0);
        };
        // One group with every path is fastest when it fits (measured on the
        // NequIP-like graph: fewer launches and index loads, the g row read in
        // one pass); larger problems are split so that no group spills.
        auto make_groups = [&](bool dbl, std::vector<Group> &groups, int &waves) {
            // split budget of the register estimate (measured on the MACE-like plan, first-order
            // backward: fp32 at 140 gives six groups that need 232 VGPRs and no spill, 20.75 ms,
            // against 256 VGPRs, a 128-byte spill and 21.8 ms at 168, and five spilling groups
            // above 176; fp64 at 200 gives 11 groups at 247 VGPRs, two waves per SIMD and
            // 38.8 ms, against 17 groups and 46.6 ms at 168, 56.8 ms at 140, and one wave per SIMD
            // from 216 on (8 groups at 230: 48.1 ms); with the rolling prefetch below 180 fits it in
            // 247 VGPRs: 38.1 against 38.7 ms).  The double backward's sender pass keeps 168.
            const int split_budget =
                getenv_int("CGTP_BWD_BUDGET", dbl ? 168 : P.dtype == CGTP_F64 ? 180 : 140);
            const int one_group_limit = 200;
            groups.clear();
            std::vector<int> all_paths;
            for (int i = 0; i < (int)P.paths.size(); ++i) all_paths.push_back(i);
            bool split = estimate(all_paths, false, dbl) > one_group_limit;
            if (const char *e = std::getenv(dbl ? "CGTP_DBL_SPLIT" : "CGTP_BWD_SPLIT")) split = std::atoi(e) != 0;
            if (!split) {
                Group all;
                all.paths = all_paths;
                groups.push_back(all);
            }
            for (int b = 0; split && b < (int)P.sh.size(); ++b) {
                Group cur;
                for (int i = 0; i < (int)P.paths.size(); ++i) {
                    if (P.paths[i].i2 != b) continue;
                    std::vector<int> trial = cur.paths;
                    trial.push_back(i);
                    if (!cur.paths.empty() && estimate(trial, false, dbl) > split_budget) {
                        groups.push_back(cur);
                        cur = Group();
                    }
                    cur.paths.push_back(i);
                }
                if (!cur.paths.empty()) groups.push_back(cur);
            }
            int est_max = 0;
            for (Group &g : groups) {
                for (int pi : g.paths) g.mul = std::max(g.mul, P.paths[pi].mul_in);
                finish_group(g);
                // register double-buffering measured slower (it lowers occupancy and the
                // backward is bound by outstanding L1 misses, not by issue latency)
                g.prefetch = !dbl && P.bwd_prefetch > 0;
                est_max = std::max(est_max, estimate(g.paths, g.prefetch, dbl));
            }
            waves = std::max(1, std::min(4, 512 * 4 / (5 * std::max(est_max, 1))));
        };
        make_groups(false, P.bwd_groups, P.bwd_waves_per_eu);
        make_groups(P.mode == CGTP_UVU, P.dbl_groups, P.dbl_bwd_waves_per_eu);
        if (P.mode != CGTP_UVU) P.dbl_groups.clear();
    }

    // Occupancy targets: 4 waves per SIMD (<= 128 VGPRs) keeps enough loads in
    // flight to cover HBM latency in the forward (fp64 doubles the register
    // need and gets 2); the backward target follows its register estimate.
    // CGTP_FWD_WAVES / CGTP_BWD_WAVES override (tuning).
    P.fwd_waves_per_eu = P.dtype == CGTP_F64 ? 2 : 4;
    if (const char *e = std::getenv("CGTP_FWD_WAVES")) P.fwd_waves_per_eu = std::max(1, std::atoi(e));
    if (const char *e = std::getenv("CGTP_FWD_ROW_SPLIT")) {
        const int v = std::atoi(e);
        P.fwd_row_split = (v == 1 || v == 2 || v == 4) ? v : 0;
    }
    // the double backward's receiver pass holds twice the forward's operands
    P.dbl_fwd_waves_per_eu = std::max(1, P.fwd_waves_per_eu / 2);
    if (const char *e = std::getenv("CGTP_DBL_FWD_WAVES")) P.dbl_fwd_waves_per_eu = std::max(1, std::atoi(e));
    if (const char *e = std::getenv("CGTP_DBL_BWD_WAVES")) P.dbl_bwd_waves_per_eu = std::max(1, std::atoi(e));
    if (const char *e = std::getenv("CGTP_BWD_WAVES")) P.bwd_waves_per_eu = std::max(1, std::atoi(e));
    P.rbw_waves_per_eu = 2;
    if (const char *e = std::getenv("CGTP_RBW_WAVES")) P.rbw_waves_per_eu = std::max(1, std::atoi(e));
    if (const char *e = std::getenv("CGTP_RBW_SCHED_BARRIER")) P.rbw_sched_barrier = std::atoi(e) != 0;
    if (const char *e = std::getenv("CGTP_RBW_PREFETCH")) P.rbw_prefetch = std::atoi(e) != 0;
    P.uvw_waves_per_eu = P.dtype == CGTP_F64 ? 1 : 2;
    if (const char *e = std::getenv("CGTP_UVC_RPW")) P.uvc_rpw = std::atoi(e) >= 4 ? 4 : std::atoi(e) >= 2 ? 2 : 1;
    P.uvc_waves_per_eu = 4 / P.uvc_rpw;  // the workgroup's 16 / rpw waves spread over 4 SIMDs
    if (const char *e = std::getenv("CGTP_UVW_WAVES")) P.uvw_waves_per_eu = std::max(1, std::atoi(e));
    if (const char *e = std::getenv("CGTP_UVB_W_WAVES")) P.uvb_w_waves_per_eu = std::max(1, std::atoi(e));
    if (const char *e = std::getenv("CGTP_UVB_W_PREFETCH")) P.uvb_w_prefetch = std::max(1, std::min(8, std::atoi(e)));
    if (const char *e = std::getenv("CGTP_UVB_W_PIPELINE")) P.uvb_w_pipeline = std::atoi(e) != 0;
    // the staged gradient blocks hold one path's block per lane in registers (64 values at l = 7):
    // fp32 only (fp64 doubles that)
    P.uvb_w_stage = P.dtype == CGTP_F32;
    if (const char *e = std::getenv("CGTP_UVB_W_STAGE")) P.uvb_w_stage = std::atoi(e) != 0;
    if (const char *e = std::getenv("CGTP_UVB_XY_PREFETCH")) P.uvb_xy_prefetch = std::max(1, std::min(8, std::atoi(e)));
    if (const char *e = std::getenv("CGTP_BWD_SCHED_BARRIER")) P.bwd_sched_barrier = std::atoi(e) != 0;
    // Rolling prefetch in the first-order sender pass pays where the plan is split into several
    // path groups (MACE-like graph: fp32 20.1 -> 17.6 ms; fp64 at the split budget of 180 38.7 ->
    // 38.1 ms); single-group plans lose occupancy to the extra live range (NequIP-like graph: 0.30
    // -> 0.68 ms, streaming graph: 29.1 -> 30.6 ms).
    P.bwd_rolling = P.bwd_groups.size() > 1 ? 1 : 0;
    if (const char *e = std::getenv("CGTP_BWD_ROLLING")) P.bwd_rolling = std::atoi(e);
    if (const char *e = std::getenv("CGTP_PERMLANE_SUMS")) P.permlane_sums = std::atoi(e) != 0;
    // Pinning the receiver pass's next-edge loads ahead of the arithmetic pays for plans split into
    // several path groups, whose long per-edge arithmetic hides a whole load latency (MACE-like
    // graph: fp32 4.27 -> 4.09 ms, fp64 9.52 -> 9.23 ms); single-group plans keep four waves per
    // SIMD without it, and with it spill (NequIP-like graph: 107 -> 142 us).
    P.fwd_sched_barrier = P.fwd_groups.size() > 1;
    if (const char *e = std::getenv("CGTP_FWD_SCHED_BARRIER")) P.fwd_sched_barrier = std::atoi(e) != 0;
    // Single-group plans split rows over 2 or 4 waves on graphs with few receivers against the wave
    // slots; the barrier pays there and not on large graphs (one wave per row), so those kernels
    // alone take it (NequIP-like graph: 102 -> 97 us; the 10M-edge plan on a 5,000-node graph 0.59
    // -> 0.44 ms; on 200,000-node graphs 4.61 -> 4.64 and 9.82 -> 10.04 ms with it everywhere).
    // Split plans' receiver passes take two edges per loop iteration with alternating operand sets
    // (no operand copies; MACE-like graph: fp32 4.02 -> 4.00 ms, fp64 8.98 -> 8.86-8.95 ms; the
    // single-group plans measured the same either way and keep one)
    P.fwd_unroll = P.fwd_sched_barrier ? 2 : 1;
    if (const char *e = std::getenv("CGTP_FWD_UNROLL")) P.fwd_unroll = std::atoi(e) > 1 ? 2 : 1;
    if (const char *e = std::getenv("CGTP_SPLIT_SCHED_BARRIER")) P.split_sched_barrier = std::atoi(e) != 0;
    // with the barrier those kernels need a few registers more than four waves allow in fp32 (the
    // NequIP-like plan: 134 and no spill at three, a 7-register spill at four)
    P.split_fwd_waves = P.dtype == CGTP_F32 && P.fwd_waves_per_eu == 4 ? 3 : 0;
    if (const char *e = std::getenv("CGTP_SPLIT_FWD_WAVES")) P.split_fwd_waves = std::max(0, std::atoi(e));
    // With the next edge's operands pinned ahead, the fp32 receiver pass of a split plan needs a few
    // registers more than four waves per SIMD allow (MACE-like graph: 128 VGPRs and a 6-register
    // spill at 4, 130 and none at 3: 4.07 against 4.03-4.04 ms, alternating runs on one box).
    P.conv_fwd_waves = P.dtype == CGTP_F32 && P.fwd_sched_barrier && P.fwd_waves_per_eu == 4 ? 3 : 0;
    if (const char *e = std::getenv("CGTP_CONV_FWD_WAVES")) P.conv_fwd_waves = std::max(0, std::atoi(e));
    if (const char *e = std::getenv("CGTP_UVC_SCHED_BARRIER")) P.uvc_sched_barrier = std::atoi(e) != 0;
}

// Internal plan of the uvw convolution backward: the paths and CG blocks of P, each path
// feeding an output block of its own (mul_in x l3, in path order), uvu with unit weights.  Its
// sender pass, given G_p = W_p^T g as the output gradient, yields the input and SH gradients.
std::unique_ptr<Plan> make_conv_uvw_aux(const Plan &P)
{
    auto A = std::make_unique<Plan>();
    A->mode = CGTP_UVU;
    A->dtype = P.dtype;
    A->ins = P.ins;
    A->sh = P.sh;
    A->paths = P.paths;
    int off = 0;
    int64_t w = 0;
    for (size_t i = 0; i < A->paths.size(); ++i) {
        Path &p = A->paths[i];
        Irrep ir;
        ir.mul = p.mul_in;
        ir.l = p.l3;
        ir.p = p.p3;
        A->out.push_back(ir);
        p.slot = (int)i;
        p.o = off;
        p.mul_out = p.mul_in;
        p.w_off = w;
        off += ir.dim();
        w += p.mul_in;
    }
    A->d_x = P.d_x;
    A->d_sh = P.d_sh;
    A->d_out = off;
    A->w_numel = w;
    A->nnz_total = P.nnz_total;
    A->unit_weights = true;
    schedule(*A);
    return A;
}

}  // namespace cgtp
