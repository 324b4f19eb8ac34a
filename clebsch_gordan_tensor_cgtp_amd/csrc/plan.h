// Internal plan representation shared by the planner, the code generator and
// the ABI layer of libcgtp.  Nothing here is visible through include/cgtp.h.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <stdexcept>
#include <string>
#include <vector>

#include "cgtp.h"

namespace cgtp {

// An error with a status code; converted to cgtp_status at the ABI edge.
struct Error : std::runtime_error {
    cgtp_status code;
    Error(cgtp_status c, const std::string &m) : std::runtime_error(m), code(c) {}
};

struct Irrep {
    int mul = 0, l = 0, p = 1;
    int dim() const { return mul * (2 * l + 1); }
};

struct Nonzero {
    int i, j, k;
    double c;
};

struct Path {
    int i1, i2, slot;
    int l1, l2, l3, p3;
    int a, b, o;           // offsets of the x, y and out blocks
    int mul_in, mul_out;
    int64_t w_off;
    std::vector<Nonzero> nz;
};

// Work split of one generated kernel: a set of paths handled by one wave.
struct Group {
    std::vector<int> paths;  // indices into Plan::paths, canonical order
    int mul = 0;             // channels of every path in the group
    int ct = 64;             // lanes per edge slot (power of two <= 64)
    int es = 1;              // edge slots per wave = 64 / ct
    int tiles = 1;           // channel tiles of width ct covering mul
    bool prefetch = false;   // backward: double-buffer the next edge's operands in registers
    int part = 0;            // batched uvw dx/dY: 0 the whole input block, 1 / 2 the halves of a split one
};

struct Plan {
    std::vector<Irrep> ins, sh, out;
    cgtp_mode mode = CGTP_UVU;
    cgtp_dtype dtype = CGTP_F32;
    std::vector<Path> paths;
    int d_x = 0, d_sh = 0, d_out = 0;
    int64_t w_numel = 0;
    int nnz_total = 0;

    std::vector<Group> fwd_groups;  // forward: one wave per (receiver, group, tile)
    std::vector<Group> rbw_groups;  // receiver-order backward: one launch per group, in order
    int fwd_tasks = 0;              // sum over groups of tiles
    std::vector<Group> bwd_groups;  // backward: one launch per group, in order
    std::vector<Group> uvw_groups;  // uvw batched product: one launch per group of output slots
    std::vector<Group> dbl_groups;  // double backward, sender pass: one launch per group, in order
    std::vector<Group> uvc_groups;  // uvw convolution: one launch per group, in order (a slot may span groups)
    std::vector<Group> uvb_x_groups;  // uvw batched backward, dx/dy: one input block per group (launched in order)
    std::vector<Group> uvb_w_groups;  // uvw batched backward, dW partials: up to 16 paths per group
    bool uvb_ok = false;            // uvw batched backward supported (every mul_in, mul_out <= 16)
    bool uvc_ok = false;            // uvw convolution supported (every path group's T staging fits LDS)
    std::string uvc_why;            // why not, when uvc_ok is false
    bool unit_weights = false;      // internal plans: every weight is 1 (not read), only the sender pass
    int fwd_waves_per_eu = 4;       // occupancy target given to the compiler (min waves per SIMD)
    int conv_fwd_waves = 0;         // the convolution's receiver pass, when it differs (0: fwd_waves_per_eu)
    int split_fwd_waves = 0;        // its row-split kernels, when they differ (0: as the receiver pass)
    int bwd_waves_per_eu = 4;
    int uvw_waves_per_eu = 2;
    int dbl_fwd_waves_per_eu = 2;   // double backward, receiver pass (twice the forward's operands)
    int dbl_bwd_waves_per_eu = 2;   // double backward, sender pass
    int rbw_waves_per_eu = 2;       // backward in receiver order (cgtp_conv_rbw)
    int uvc_waves_per_eu = 2;       // uvw convolution
    int uvb_w_waves_per_eu = 1;     // uvw batched backward, dW kernel
    int uvb_w_prefetch = 2;         // uvw batched backward, dW kernel: (path, k) blocks of gradients in flight
    bool uvb_w_pipeline = true;     // uvw batched backward, dW kernel: a block's MFMAs issued during the next block
    bool uvb_w_stage = true;        // uvw batched backward, dW kernel: per-path gradient blocks staged in LDS
    int uvb_xy_prefetch = 2;        // uvw batched backward, dx/dY kernel: (path, k) blocks of gradients in flight
    int uvc_rpw = 4;                // uvw convolution: receivers per wave (16 / waves per workgroup)
    bool stream_hint = true;        // nontemporal loads/stores for once-touched per-edge rows
    bool scalar_wave = true;        // wave index read from the first lane (uniform, SGPR-held)
    bool permlane_sums = true;      // lane sums over xor 16 / 32 by v_permlane*_swap instead of shuffles
    int fwd_unroll = 1;             // receiver pass: edges per loop iteration (2: operand sets alternate, no copies)
    bool bwd_sched_barrier = true;  // keep path blocks of the backward from interleaving
    int bwd_rolling = 0;            // sender pass: next edge's operands loaded as this edge frees them (2: pinned by barriers)
    bool fwd_sched_barrier = false; // keep the receiver pass's next-edge loads ahead of its arithmetic
    bool split_sched_barrier = true; // the same in the row-split forward kernels of single-group plans
    bool uvc_sched_barrier = true;  // the same in the uvw convolution's edge stream
    bool rbw_sched_barrier = true;  // the same for the receiver-order backward, per path
    bool rbw_prefetch = false;      // receiver-order backward: sender ids two edges ahead, operands one ahead
    int bwd_prefetch = -1;          // -1: per group by register estimate; 0/1 forced
    bool fwd_split_inputs = false;  // forward groups follow input-irrep classes (measured slower)
    int fwd_row_split = 0;          // receiver-owned passes: waves per row forced (1, 2, 4); 0 = by N
    std::string source;             // generated HIP source
    std::vector<char> code;         // compiled gfx950 code object

    std::mutex mu;                  // guards the per-device module table
    struct Loaded {
        hipModule_t module = nullptr;
        hipFunction_t conv_fwd = nullptr, conv_bwd = nullptr, tp_fwd = nullptr, tp_uvw = nullptr;
        hipFunction_t dbwd_recv = nullptr, dbwd_send = nullptr, conv_uvw = nullptr, tp_bwd = nullptr;
        hipFunction_t rbw = nullptr, rbw_dx = nullptr;  // backward in receiver order and its dx sum
        // receiver rows split over 2 / 4 waves (single-task plans; else null)
        hipFunction_t conv_fwd_split[2] = {nullptr, nullptr}, dbwd_recv_split[2] = {nullptr, nullptr};
    };
    std::map<int, Loaded> loaded;

    // Radial projection, one module per number of radial features R (built on first use): the
    // forward, the backward's sender pass (dx, dY, drho, dTheta partials) and their reduction.
    struct Radial {
        std::string source;
        std::vector<char> code;
        std::vector<Group> bwd_groups;  // sender-pass groups of the backward (R-dependent)
        struct Fns {
            hipModule_t module = nullptr;
            hipFunction_t fwd = nullptr, bwd = nullptr, reduce = nullptr;
        };
        std::map<int, Fns> loaded;  // per device
    };
    std::map<int, Radial> radial;

    // uvw batched backward: its own module, built on first use (large at high L).
    struct UvwBackward {
        std::string source;
        std::vector<char> code;
        struct Fns {
            hipModule_t module = nullptr;
            hipFunction_t xy = nullptr, w = nullptr, reduce = nullptr;
        };
        std::map<int, Fns> loaded;  // per device
    } uvb;

    // uvw convolution backward: G = W^T g per receiver and the dW partials (own module, built
    // on first use), and the sender pass of an internal uvu plan with one output block per path
    // and unit weights, which turns G into dx and dY.
    struct ConvUvwBackward {
        std::string source;
        std::vector<char> code;
        struct Fns {
            hipModule_t module = nullptr;
            hipFunction_t g = nullptr, w = nullptr, reduce = nullptr;
            hipFunction_t fwd_acc = nullptr;  // the forward, adding to its output (double backward)
            hipFunction_t fwd_rad = nullptr;  // the forward for one radial channel (radial projection)
        };
        std::map<int, Fns> loaded;  // per device
    } ucb;
    std::unique_ptr<Plan> aux;
};

// planner.cpp
std::vector<Irrep> parse_irreps(const std::string &text, const char *what);
void build_paths(Plan &plan);
std::vector<Nonzero> real_cg_nonzeros(int l1, int l2, int l3);
void schedule(Plan &plan);

// codegen.cpp
std::string generate_source(const Plan &plan);
std::string generate_radial_source(const Plan &plan, int R, const std::vector<Group> &bwd_groups, int bwd_waves);
bool radial_bwd_fits(const Plan &plan, int R, const std::vector<Group> &bwd_groups);
// LDS bytes of the radial forward's Theta copy (one path group's channel tile) and whether it fits
long radial_fwd_lds_bytes(const Plan &plan, int R);
bool radial_fwd_fits(const Plan &plan, int R);

// jit.cpp
void compile_module(Plan &plan);
std::vector<char> compile_source(const std::string &source);
const Plan::Loaded &module_for_current_device(Plan &plan);
const Plan::Radial::Fns &radial_functions_for_current_device(Plan &plan, int R);
const std::vector<Group> &radial_bwd_groups_of(Plan &plan, int R);
const std::string &prepare_radial(Plan &plan, int R);
std::string generate_uvw_backward_source(const Plan &plan);
const std::string &prepare_uvw_backward(Plan &plan);
const Plan::UvwBackward::Fns &uvw_backward_for_current_device(Plan &plan);
std::string generate_conv_uvw_backward_source(const Plan &plan);
const Plan::ConvUvwBackward::Fns &conv_uvw_backward_for_current_device(Plan &plan);
Plan &conv_uvw_aux_plan(Plan &plan);
const std::string &prepare_conv_uvw_backward(Plan &plan);
std::unique_ptr<Plan> make_conv_uvw_aux(const Plan &plan);
std::vector<Group> radial_bwd_groups(const Plan &plan, int R, int &waves_per_eu);
void unload_modules(Plan &plan);
int64_t conv_uvw_g_width(const Plan &plan);
// accumulators per lane of forward path group gi (the LDS words per lane of one split part)
int fwd_group_accs(const Plan &plan, int gi);
// whether the receiver-owned passes may split a receiver row over several waves
bool fwd_splittable(const Plan &plan);
// batched uvw forward: 16-wide tiles of output channels (one wave per tile and 16-row block)
int uvw_out_tiles(const Plan &plan);
int conv_uvw_g_items(const Plan &plan, std::vector<std::pair<int, int>> *items);

}  // namespace cgtp
