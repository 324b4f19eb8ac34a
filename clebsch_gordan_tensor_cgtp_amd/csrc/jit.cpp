// hipRTC compilation of the generated module for gfx950, an on-disk
// content-addressed cache of code objects, and per-device module loading.
//
// sciencestack.ai page (TL;DR, Abstract): the kernels are generated and
// JIT-compiled per model configuration.  Here the compiler is hipRTC, the
// target is fixed to gfx950, and packed fp32 instructions are disabled.
#include <dlfcn.h>
#include <hip/hiprtc.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <climits>
#include <cstring>
#include <type_traits>
#include <fstream>
#include <sstream>

#include "plan.h"

namespace cgtp {

static const char *const kOptions[] = {
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
};

static uint64_t fnv1a(const std::string &s, uint64_t h)
{
    for (unsigned char c : s) {
        h ^= c;
        h *= 1099511628211ull;
    }
    return h;
}

static std::string cache_dir()
{
    const char *env = std::getenv("CGTP_CACHE_DIR");
    if (env && *env) return env;
    Dl_info info;
    if (dladdr(reinterpret_cast<void *>(&cache_dir), &info) && info.dli_fname) {
        std::string p = info.dli_fname;
        size_t slash = p.rfind('/');
        if (slash != std::string::npos) return p.substr(0, slash) + "/jit_cache";
    }
    return "jit_cache";
}

static bool read_file(const std::string &path, std::vector<char> &out)
{
    std::ifstream f(path, std::ios::binary);
    if (!f) return false;
    out.assign(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
    return out.size() > 4 && std::memcmp(out.data(), "\x7f" "ELF", 4) == 0;
}

static void write_file_atomic(const std::string &path, const std::vector<char> &data)
{
    std::string tmp = path + ".tmp" + std::to_string(::getpid());
    {
        std::ofstream f(tmp, std::ios::binary);
        if (!f) return;
        f.write(data.data(), (std::streamsize)data.size());
        if (!f) return;
    }
    std::rename(tmp.c_str(), path.c_str());
}

// The compiler.  A host process may already hold another hipRTC and code-object compiler
// than the ROCm installation's (a framework loaded first can bring its own copies, and a
// library with the same soname is then shared by everyone); their code for the same source can
// differ (measured: a register spill in one and not the other).  So the installation's hipRTC is
// loaded in a link namespace of its own (dlmopen), where it also finds the installation's
// compiler library, and the cache key names the compiler that made each code object.  If that
// load fails, the hipRTC the library was linked against is used.
struct Rtc {
    decltype(&hiprtcCreateProgram) create = hiprtcCreateProgram;
    decltype(&hiprtcCompileProgram) compile = hiprtcCompileProgram;
    decltype(&hiprtcGetProgramLogSize) log_size = hiprtcGetProgramLogSize;
    decltype(&hiprtcGetProgramLog) log = hiprtcGetProgramLog;
    decltype(&hiprtcGetCodeSize) code_size = hiprtcGetCodeSize;
    decltype(&hiprtcGetCode) code = hiprtcGetCode;
    decltype(&hiprtcDestroyProgram) destroy = hiprtcDestroyProgram;
    decltype(&hiprtcGetErrorString) error_string = hiprtcGetErrorString;
    decltype(&hiprtcVersion) version = hiprtcVersion;
    std::string identity;  // which library compiles, for the cache key
    // The C library of the private link namespace keeps its own `environ`, copied when the
    // namespace was created.  A later setenv/putenv in the process may move the environment
    // array and free the old one, leaving that copy dangling (hipRTC reads the environment):
    // it is pointed at the process's current array before every call into hipRTC.
    char ***ns_environ = nullptr;
};

extern "C" char **environ;

static std::string real_path_of(void *sym)
{
    Dl_info info;
    if (!dladdr(sym, &info) || !info.dli_fname) return "unknown";
    char buf[4096];
    return ::realpath(info.dli_fname, buf) ? std::string(buf) : std::string(info.dli_fname);
}

static const Rtc &rtc()
{
    static const Rtc r = [] {
        Rtc x;
        std::string path;
        if (const char *e = std::getenv("CGTP_HIPRTC")) {
            path = e;
        } else {
            const char *root = std::getenv("ROCM_PATH");
            path = std::string(root && *root ? root : "/opt/rocm") + "/lib/libhiprtc.so.7";
        }
        void *h = path.empty() ? nullptr : ::dlmopen(LM_ID_NEWLM, path.c_str(), RTLD_NOW | RTLD_LOCAL);
        bool ok = h != nullptr;
        auto get = [&](auto &fn, const char *name) {
            if (!ok) return;
            void *p = ::dlsym(h, name);
            if (p)
                fn = reinterpret_cast<std::remove_reference_t<decltype(fn)>>(p);
            else
                ok = false;
        };
        Rtc y;
        get(y.create, "hiprtcCreateProgram");
        get(y.compile, "hiprtcCompileProgram");
        get(y.log_size, "hiprtcGetProgramLogSize");
        get(y.log, "hiprtcGetProgramLog");
        get(y.code_size, "hiprtcGetCodeSize");
        get(y.code, "hiprtcGetCode");
        get(y.destroy, "hiprtcDestroyProgram");
        get(y.error_string, "hiprtcGetErrorString");
        get(y.version, "hiprtcVersion");
        if (ok) {
            Lmid_t lmid;
            if (::dlinfo(h, RTLD_DI_LMID, &lmid) == 0)
                if (void *libc = ::dlmopen(lmid, "libc.so.6", RTLD_NOW | RTLD_NOLOAD))
                    y.ns_environ = static_cast<char ***>(::dlsym(libc, "environ"));
            x = y;
        } else if (h) {
            ::dlclose(h);
        }
        x.identity = real_path_of(reinterpret_cast<void *>(x.create));
        int major = 0, minor = 0;
        x.version(&major, &minor);
        x.identity += " " + std::to_string(major) + "." + std::to_string(minor);
        if (std::getenv("CGTP_LOG")) std::fprintf(stderr, "[cgtp] compiler: %s\n", x.identity.c_str());
        return x;
    }();
    return r;
}

void compile_module(Plan &P) { P.code = compile_source(P.source); }

std::vector<char> compile_source(const std::string &source)
{
    std::vector<char> code;
    const Rtc &R = rtc();
    std::string opts;
    for (const char *o : kOptions) opts += std::string(o) + " ";
    std::string key_src = source + "\n//" + opts + R.identity;
    char name[64];
    std::snprintf(name, sizeof name, "cgtp_%016llx%016llx.hsaco",
                  (unsigned long long)fnv1a(key_src, 1469598103934665603ull),
                  (unsigned long long)fnv1a(key_src, 0x9e3779b97f4a7c15ull));
    const std::string dir = cache_dir();
    const std::string path = dir + "/" + name;
    if (read_file(path, code)) return code;

    hiprtcProgram prog;
    if (R.ns_environ && R.ns_environ != &environ) *R.ns_environ = environ;
    if (R.create(&prog, source.c_str(), "cgtp_module.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS)
        throw Error(CGTP_ERR_COMPILE, "hiprtcCreateProgram failed");
    hiprtcResult rc = R.compile(prog, (int)(sizeof kOptions / sizeof kOptions[0]), kOptions);
    if (rc != HIPRTC_SUCCESS) {
        size_t n = 0;
        R.log_size(prog, &n);
        std::string log(n, '\0');
        if (n) R.log(prog, &log[0]);
        R.destroy(&prog);
        throw Error(CGTP_ERR_COMPILE, std::string("hipRTC: ") + R.error_string(rc) + "\n" + log);
    }
    size_t n = 0;
    R.code_size(prog, &n);
    code.resize(n);
    R.code(prog, code.data());
    R.destroy(&prog);
    ::mkdir(dir.c_str(), 0755);
    write_file_atomic(path, code);
    return code;
}

static void check(hipError_t e, const char *what)
{
    if (e != hipSuccess) throw Error(CGTP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

const Plan::Loaded &module_for_current_device(Plan &P)
{
    int dev = 0;
    check(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(P.mu);
    auto it = P.loaded.find(dev);
    if (it != P.loaded.end()) return it->second;
    Plan::Loaded L;
    check(hipModuleLoadData(&L.module, P.code.data()), "hipModuleLoadData");
    if (P.unit_weights) {
        check(hipModuleGetFunction(&L.conv_bwd, L.module, "cgtp_conv_uvw_bwd_xy"), "hipModuleGetFunction(uvw_bwd_xy)");
    } else if (P.mode == CGTP_UVU) {
        check(hipModuleGetFunction(&L.conv_fwd, L.module, "cgtp_conv_fwd"), "hipModuleGetFunction(conv_fwd)");
        check(hipModuleGetFunction(&L.conv_bwd, L.module, "cgtp_conv_bwd"), "hipModuleGetFunction(conv_bwd)");
        check(hipModuleGetFunction(&L.tp_fwd, L.module, "cgtp_tp_fwd"), "hipModuleGetFunction(tp_fwd)");
        check(hipModuleGetFunction(&L.dbwd_recv, L.module, "cgtp_conv_dbwd_recv"), "hipModuleGetFunction(dbwd_recv)");
        check(hipModuleGetFunction(&L.dbwd_send, L.module, "cgtp_conv_dbwd_send"), "hipModuleGetFunction(dbwd_send)");
        if (fwd_splittable(P)) {
            check(hipModuleGetFunction(&L.conv_fwd_split[0], L.module, "cgtp_conv_fwd_split2"), "hipModuleGetFunction");
            check(hipModuleGetFunction(&L.conv_fwd_split[1], L.module, "cgtp_conv_fwd_split4"), "hipModuleGetFunction");
            check(hipModuleGetFunction(&L.dbwd_recv_split[0], L.module, "cgtp_conv_dbwd_recv_split2"),
                  "hipModuleGetFunction");
            check(hipModuleGetFunction(&L.dbwd_recv_split[1], L.module, "cgtp_conv_dbwd_recv_split4"),
                  "hipModuleGetFunction");
        }
        check(hipModuleGetFunction(&L.tp_bwd, L.module, "cgtp_tp_bwd"), "hipModuleGetFunction(tp_bwd)");
        check(hipModuleGetFunction(&L.rbw, L.module, "cgtp_conv_rbw"), "hipModuleGetFunction(conv_rbw)");
        check(hipModuleGetFunction(&L.rbw_dx, L.module, "cgtp_conv_rbw_dx"), "hipModuleGetFunction(conv_rbw_dx)");
    } else {
        check(hipModuleGetFunction(&L.tp_uvw, L.module, "cgtp_tp_uvw"), "hipModuleGetFunction(tp_uvw)");
        check(hipModuleGetFunction(&L.conv_uvw, L.module, "cgtp_conv_uvw"), "hipModuleGetFunction(conv_uvw)");

    }
    return P.loaded.emplace(dev, L).first->second;
}

// Generate and compile the radial module for R (no device needed); caller holds P.mu.
static Plan::Radial &radial_locked(Plan &P, int R)
{
    Plan::Radial &rv = P.radial[R];
    if (rv.code.empty()) {
        int waves = 1;
        rv.bwd_groups = radial_bwd_groups(P, R, waves);
        rv.source = generate_radial_source(P, R, rv.bwd_groups, waves);
        rv.code = compile_source(rv.source);
    }
    return rv;
}

const std::vector<Group> &radial_bwd_groups_of(Plan &P, int R)
{
    std::lock_guard<std::mutex> lock(P.mu);
    return radial_locked(P, R).bwd_groups;
}

const std::string &prepare_radial(Plan &P, int R)
{
    std::lock_guard<std::mutex> lock(P.mu);
    return radial_locked(P, R).source;
}

const Plan::Radial::Fns &radial_functions_for_current_device(Plan &P, int R)
{
    int dev = 0;
    check(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(P.mu);
    Plan::Radial &rv = radial_locked(P, R);
    auto it = rv.loaded.find(dev);
    if (it != rv.loaded.end()) return it->second;
    Plan::Radial::Fns F;
    check(hipModuleLoadData(&F.module, rv.code.data()), "hipModuleLoadData");
    if (radial_fwd_fits(P, R))
        check(hipModuleGetFunction(&F.fwd, F.module, "cgtp_conv_fwd_radial"), "hipModuleGetFunction(conv_fwd_radial)");
    if (radial_bwd_fits(P, R, rv.bwd_groups)) {
        check(hipModuleGetFunction(&F.bwd, F.module, "cgtp_conv_bwd_radial"), "hipModuleGetFunction(conv_bwd_radial)");
        check(hipModuleGetFunction(&F.reduce, F.module, "cgtp_reduce_chunks"), "hipModuleGetFunction(reduce)");
    }
    return rv.loaded.emplace(dev, F).first->second;
}

}  // namespace cgtp

namespace cgtp {

static void uvb_locked(Plan &P)
{
    if (P.uvb.code.empty()) {
        P.uvb.source = generate_uvw_backward_source(P);
        P.uvb.code = compile_source(P.uvb.source);
    }
}

const std::string &prepare_uvw_backward(Plan &P)
{
    std::lock_guard<std::mutex> lock(P.mu);
    uvb_locked(P);
    return P.uvb.source;
}

const Plan::UvwBackward::Fns &uvw_backward_for_current_device(Plan &P)
{
    int dev = 0;
    check(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(P.mu);
    uvb_locked(P);
    auto it = P.uvb.loaded.find(dev);
    if (it != P.uvb.loaded.end()) return it->second;
    Plan::UvwBackward::Fns F;
    check(hipModuleLoadData(&F.module, P.uvb.code.data()), "hipModuleLoadData");
    check(hipModuleGetFunction(&F.xy, F.module, "cgtp_tp_uvw_bwd_xy"), "hipModuleGetFunction(uvw_bwd_xy)");
    check(hipModuleGetFunction(&F.w, F.module, "cgtp_tp_uvw_bwd_w"), "hipModuleGetFunction(uvw_bwd_w)");
    check(hipModuleGetFunction(&F.reduce, F.module, "cgtp_reduce_chunks"), "hipModuleGetFunction(reduce)");
    return P.uvb.loaded.emplace(dev, F).first->second;
}

// uvw convolution backward: the G / dW module and the internal sender-pass plan; caller holds P.mu
static void ucb_locked(Plan &P)
{
    if (P.ucb.code.empty()) {
        P.ucb.source = generate_conv_uvw_backward_source(P);
        P.ucb.code = compile_source(P.ucb.source);
    }
    if (!P.aux) {
        std::unique_ptr<Plan> A = make_conv_uvw_aux(P);
        A->source = generate_source(*A);
        A->code = compile_source(A->source);
        P.aux = std::move(A);
    }
}

const std::string &prepare_conv_uvw_backward(Plan &P)
{
    std::lock_guard<std::mutex> lock(P.mu);
    ucb_locked(P);
    return P.ucb.source;
}

Plan &conv_uvw_aux_plan(Plan &P)
{
    std::lock_guard<std::mutex> lock(P.mu);
    ucb_locked(P);
    return *P.aux;
}

const Plan::ConvUvwBackward::Fns &conv_uvw_backward_for_current_device(Plan &P)
{
    int dev = 0;
    check(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(P.mu);
    ucb_locked(P);
    auto it = P.ucb.loaded.find(dev);
    if (it != P.ucb.loaded.end()) return it->second;
    Plan::ConvUvwBackward::Fns F;
    check(hipModuleLoadData(&F.module, P.ucb.code.data()), "hipModuleLoadData");
    check(hipModuleGetFunction(&F.g, F.module, "cgtp_conv_uvw_bwd_g"), "hipModuleGetFunction(conv_uvw_bwd_g)");
    check(hipModuleGetFunction(&F.w, F.module, "cgtp_conv_uvw_bwd_w"), "hipModuleGetFunction(conv_uvw_bwd_w)");
    check(hipModuleGetFunction(&F.reduce, F.module, "cgtp_reduce_chunks"), "hipModuleGetFunction(reduce)");
    check(hipModuleGetFunction(&F.fwd_acc, F.module, "cgtp_conv_uvw_acc"), "hipModuleGetFunction(conv_uvw_acc)");
    check(hipModuleGetFunction(&F.fwd_rad, F.module, "cgtp_conv_uvw_rad"), "hipModuleGetFunction(conv_uvw_rad)");
    return P.ucb.loaded.emplace(dev, F).first->second;
}

// Unload every module of the plan (and of its internal plan) on the device it was loaded on.
void unload_modules(Plan &P)
{
    std::vector<std::pair<int, hipModule_t>> mods;
    for (auto &kv : P.loaded) mods.push_back({kv.first, kv.second.module});
    for (auto &r : P.radial)
        for (auto &kv : r.second.loaded) mods.push_back({kv.first, kv.second.module});
    for (auto &kv : P.uvb.loaded) mods.push_back({kv.first, kv.second.module});
    for (auto &kv : P.ucb.loaded) mods.push_back({kv.first, kv.second.module});
    P.loaded.clear();
    for (auto &r : P.radial) r.second.loaded.clear();
    P.uvb.loaded.clear();
    P.ucb.loaded.clear();
    if (P.aux) unload_modules(*P.aux);
    if (mods.empty()) return;
    int prev = 0;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    for (auto &dm : mods)
        if (dm.second && hipSetDevice(dm.first) == hipSuccess) hipModuleUnload(dm.second);
    if (have_prev) hipSetDevice(prev);
}

}  // namespace cgtp
