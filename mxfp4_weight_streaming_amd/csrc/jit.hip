// jit.hip -- run-time compilation of the shape-templated kernels for layer
// shapes outside the ahead-of-time set, with an on-disk cache of the compiled
// code objects, and the lookup that picks a compiled-in or a loaded kernel.
//
// The pages' MoE backend compiles its kernels at run time for the actual
// matrix shapes, data types and GPU, and caches the binaries, so that a new
// shape (their 768-wide expert layer) costs seconds of compilation instead of
// an ahead-of-time build of every target ([EN] "What are the 3
// optimizations?", item 1; [ZH] "三项优化分别做了什么").  Here the same device
// headers that hipcc compiles into this library are embedded in it as text and
// handed to hipRTC with the shape as template arguments; the code object is
// written to a cache file keyed by a hash of the sources, the compile options,
// the target and the shape, and loaded with hipModuleLoadData.  Loading is
// explicit (moe_jit_load): a call with a shape that is neither compiled in nor
// loaded is rejected, never compiled behind the caller's back.
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
//   [ZH] = "NVIDIA博客:DGX Spark上三项优化使Ling-3.0-flash解码吞吐提升 42.5%"
#include <errno.h>
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "kernel_table.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

struct SourceFile {
    const char* name;
    const char* text;
};

// The device headers as text (generated at build time from csrc/).
#include "jit_sources.inc"

constexpr int kNumSources = (int)(sizeof(kJitSources) / sizeof(kJitSources[0]));
constexpr char kMagic[8] = {'M', 'O', 'E', 'J', 'I', 'T', '0', '1'};
const char* const kOptions[] = {"-O3", "-std=c++17", "-ffp-contract=fast-honor-pragmas", "-Xclang", "-target-feature",
                                "-Xclang", "-packed-fp32-ops"};
constexpr int kNumOptions = (int)(sizeof(kOptions) / sizeof(kOptions[0]));

uint64_t fnv1a(const void* data, size_t n, uint64_t h = 1469598103934665603ull)
{
    const unsigned char* p = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

uint64_t fnv1a_str(const char* s, uint64_t h) { return fnv1a(s, strlen(s) + 1, h); }

struct LoadedModule {
    int device;
    int H, I;
    bool prefer;
    hipModule_t mod;
    std::vector<KernelKey> keys;
    std::vector<hipFunction_t> fns;
};

std::mutex g_mu;                       // guards g_mods; held across compiles
std::vector<LoadedModule*> g_mods;
std::atomic<int> g_n_mods{0};
std::atomic<int> g_n_prefer{0};

const AotKernel* aot_find(const KernelKey& k)
{
    const AotKernel* tables[3] = {kGemvAot, kChunkAot, kLmHeadAot};
    const int counts[3] = {kGemvAotCount, kChunkAotCount, kLmHeadAotCount};
    for (int t = 0; t < 3; ++t)
        for (int i = 0; i < counts[t]; ++i)
            if (same_key(tables[t][i].key, k)) return &tables[t][i];
    return nullptr;
}

hipFunction_t module_find(const KernelKey& k, int device, bool want_prefer)
{
    for (const LoadedModule* m : g_mods) {
        if (m->device != device || m->prefer != want_prefer) continue;
        for (size_t i = 0; i < m->keys.size(); ++i)
            if (same_key(m->keys[i], k)) return m->fns[i];
    }
    return nullptr;
}

// Every shape-templated kernel of one (H, I) module.
std::vector<KernelKey> module_keys(int H, int I, bool chunk, bool lm)
{
    std::vector<KernelKey> keys;
    keys.push_back(key_quant(H));
    keys.push_back(key_requant(I));
    for (int mt : {1, 2, 4, 8}) {
        keys.push_back(key_router(H, mt));
        keys.push_back(key_gate_up(H, I, mt));
        keys.push_back(key_down(H, I, mt, true));
        keys.push_back(key_down(H, I, mt, false));
        if (layer_shape_ok(H, I)) keys.push_back(key_layer(H, I, mt));
    }
    if (chunk) {
        keys.push_back(key_chunk_router(H));
        keys.push_back(key_chunk_gate_up(H, I));
        keys.push_back(key_chunk_down(H, I, false));
        keys.push_back(key_chunk_down(H, I, true));
        keys.push_back(key_combine(H));
    }
    if (lm)
        for (int mt : {1, 2, 4, 8}) keys.push_back(key_lm_head(H, mt));
    return keys;
}

std::string main_source(bool chunk, bool lm)
{
    std::string s = "#include \"gemv_kernels.hpp\"\n#include \"layer_kernels.hpp\"\n";
    if (chunk) s += "#include \"chunk_kernels.hpp\"\n";
    if (lm) s += "#include \"lm_head_kernels.hpp\"\n";
    return s;
}

// Hash of everything the code object depends on.
uint64_t cache_key(int H, int I, const char* arch, bool chunk, bool lm)
{
    uint64_t h = fnv1a(kMagic, sizeof kMagic);
    for (int i = 0; i < kNumSources; ++i) {
        h = fnv1a_str(kJitSources[i].name, h);
        h = fnv1a_str(kJitSources[i].text, h);
    }
    for (int i = 0; i < kNumOptions; ++i) h = fnv1a_str(kOptions[i], h);
    int major = 0, minor = 0;
    hiprtcVersion(&major, &minor);
    const int ints[6] = {H, I, chunk ? 1 : 0, lm ? 1 : 0, major, minor};
    h = fnv1a(ints, sizeof ints, h);
    return fnv1a_str(arch, h);
}

bool make_dirs(const std::string& dir, std::string* err)
{
    std::string cur;
    size_t pos = 0;
    while (pos <= dir.size()) {
        const size_t next = dir.find('/', pos);
        cur = dir.substr(0, next == std::string::npos ? dir.size() : next);
        if (!cur.empty() && mkdir(cur.c_str(), 0755) != 0 && errno != EEXIST) {
            *err = "cannot create cache directory " + cur + ": " + strerror(errno);
            return false;
        }
        if (next == std::string::npos) break;
        pos = next + 1;
    }
    return true;
}

std::string default_cache_dir()
{
    if (const char* d = getenv("MOE_JIT_CACHE_DIR"); d != nullptr && d[0] != '\0') return d;
    if (const char* d = getenv("XDG_CACHE_HOME"); d != nullptr && d[0] != '\0') return std::string(d) + "/moe_decode_jit";
    if (const char* d = getenv("HOME"); d != nullptr && d[0] != '\0') return std::string(d) + "/.cache/moe_decode_jit";
    return "";
}

// ---- cache file ------------------------------------------------------------
// magic[8] | u64 key | u32 n | n x (i32 kind, H, I, v, u32 len, name[len]) |
// u64 code size | u64 fnv1a(code) | code
struct Entry {
    std::vector<KernelKey> keys;
    std::vector<std::string> names;   // lowered (mangled) kernel names
    std::vector<char> code;
};

template <typename T>
void put(std::vector<char>& b, const T& v)
{
    const char* p = reinterpret_cast<const char*>(&v);
    b.insert(b.end(), p, p + sizeof(T));
}

template <typename T>
bool get(const std::vector<char>& b, size_t& at, T* v)
{
    if (at + sizeof(T) > b.size()) return false;
    memcpy(v, b.data() + at, sizeof(T));
    at += sizeof(T);
    return true;
}

bool write_entry(const std::string& path, uint64_t key, const Entry& e, std::string* err)
{
    std::vector<char> b(kMagic, kMagic + sizeof kMagic);
    put(b, key);
    put(b, (uint32_t)e.keys.size());
    for (size_t i = 0; i < e.keys.size(); ++i) {
        put(b, (int32_t)e.keys[i].kind);
        put(b, (int32_t)e.keys[i].H);
        put(b, (int32_t)e.keys[i].I);
        put(b, (int32_t)e.keys[i].v);
        put(b, (uint32_t)e.names[i].size());
        b.insert(b.end(), e.names[i].begin(), e.names[i].end());
    }
    put(b, (uint64_t)e.code.size());
    put(b, fnv1a(e.code.data(), e.code.size()));
    b.insert(b.end(), e.code.begin(), e.code.end());
    // write a private temporary, then rename: readers see a whole file or none
    char tmp[64];
    snprintf(tmp, sizeof tmp, ".tmp.%d.%zx", (int)getpid(), std::hash<std::thread::id>()(std::this_thread::get_id()));
    const std::string tpath = path + tmp;
    FILE* f = fopen(tpath.c_str(), "wb");
    if (f == nullptr) {
        *err = "cannot write " + tpath + ": " + strerror(errno);
        return false;
    }
    const bool ok = fwrite(b.data(), 1, b.size(), f) == b.size();
    if (fclose(f) != 0 || !ok) {
        unlink(tpath.c_str());
        *err = "cannot write " + tpath;
        return false;
    }
    if (rename(tpath.c_str(), path.c_str()) != 0) {
        unlink(tpath.c_str());
        *err = "cannot rename the cache entry to " + path + ": " + strerror(errno);
        return false;
    }
    return true;
}

// A whole, checksummed entry for `key` holding every kernel of `keys`, or false.
bool read_entry(const std::string& path, uint64_t key, const std::vector<KernelKey>& keys, Entry* e)
{
    FILE* f = fopen(path.c_str(), "rb");
    if (f == nullptr) return false;
    std::vector<char> b;
    char buf[1 << 16];
    size_t n;
    while ((n = fread(buf, 1, sizeof buf, f)) > 0) b.insert(b.end(), buf, buf + n);
    fclose(f);
    size_t at = 0;
    if (b.size() < sizeof kMagic || memcmp(b.data(), kMagic, sizeof kMagic) != 0) return false;
    at = sizeof kMagic;
    uint64_t k = 0;
    uint32_t cnt = 0;
    if (!get(b, at, &k) || k != key || !get(b, at, &cnt) || cnt != keys.size()) return false;
    e->keys.clear();
    e->names.clear();
    for (uint32_t i = 0; i < cnt; ++i) {
        int32_t kind, H, I, v;
        uint32_t len;
        if (!get(b, at, &kind) || !get(b, at, &H) || !get(b, at, &I) || !get(b, at, &v) || !get(b, at, &len))
            return false;
        if (len == 0 || len > 4096 || at + len > b.size()) return false;
        const KernelKey kk{(KernelKind)kind, H, I, v};
        if (!same_key(kk, keys[i])) return false;
        e->keys.push_back(kk);
        e->names.emplace_back(b.data() + at, len);
        at += len;
    }
    uint64_t size = 0, sum = 0;
    if (!get(b, at, &size) || !get(b, at, &sum) || size == 0 || at + size != b.size()) return false;
    if (fnv1a(b.data() + at, size) != sum) return false;
    e->code.assign(b.data() + at, b.data() + at + size);
    return true;
}

// ---- compile -----------------------------------------------------------------
bool compile(int H, int I, const char* arch, bool chunk, bool lm, const std::vector<KernelKey>& keys, Entry* e,
             std::string* err)
{
    std::vector<const char*> hdr_text, hdr_name;
    for (int i = 0; i < kNumSources; ++i) {
        hdr_name.push_back(kJitSources[i].name);
        hdr_text.push_back(kJitSources[i].text);
    }
    const std::string src = main_source(chunk, lm);
    hiprtcProgram prog;
    hiprtcResult r = hiprtcCreateProgram(&prog, src.c_str(), "moe_jit.hip", kNumSources, hdr_text.data(),
                                         hdr_name.data());
    if (r != HIPRTC_SUCCESS) {
        *err = std::string("hiprtcCreateProgram: ") + hiprtcGetErrorString(r);
        return false;
    }
    std::vector<std::string> exprs;
    for (const KernelKey& k : keys) {
        char name[128];
        if (!kernel_expr(k, name, sizeof name)) {
            hiprtcDestroyProgram(&prog);
            *err = "internal: no name for a kernel kind";
            return false;
        }
        exprs.emplace_back(name);
        hiprtcAddNameExpression(prog, exprs.back().c_str());
    }
    std::vector<const char*> opts;
    const std::string arch_opt = std::string("--offload-arch=") + arch;
    opts.push_back(arch_opt.c_str());
    for (int i = 0; i < kNumOptions; ++i) opts.push_back(kOptions[i]);
    r = hiprtcCompileProgram(prog, (int)opts.size(), opts.data());
    if (r != HIPRTC_SUCCESS) {
        size_t n = 0;
        hiprtcGetProgramLogSize(prog, &n);
        std::string log(n, '\0');
        if (n > 0) hiprtcGetProgramLog(prog, &log[0]);
        hiprtcDestroyProgram(&prog);
        char head[96];
        snprintf(head, sizeof head, "hipRTC could not compile H=%d I=%d for %s: ", H, I, arch);
        *err = head + log;
        return false;
    }
    size_t size = 0;
    hiprtcGetCodeSize(prog, &size);
    e->code.resize(size);
    hiprtcGetCode(prog, e->code.data());
    e->keys = keys;
    e->names.clear();
    for (const std::string& x : exprs) {
        const char* lowered = nullptr;
        if (hiprtcGetLoweredName(prog, x.c_str(), &lowered) != HIPRTC_SUCCESS || lowered == nullptr) {
            hiprtcDestroyProgram(&prog);
            *err = "hipRTC has no lowered name for " + x;
            return false;
        }
        e->names.emplace_back(lowered);
    }
    hiprtcDestroyProgram(&prog);
    return true;
}

// The module's entry for (H, I) on `arch`: from the cache, else compiled and
// written to it.
JitStatus get_entry(int H, int I, const char* arch, const char* cache_dir, Entry* e, JitReport* rep, std::string* err)
{
    if (!gemv_shape_ok(H, I)) {
        char b[200];
        snprintf(b, sizeof b,
                 "(H=%d, I=%d) has no kernel geometry: needs 256 <= H <= 8192, 64 <= I <= 4096, H %% 32 == 0, "
                 "I %% 64 == 0, I %% %d == 0 and H %% %d == 0",
                 H, I, gate_up_rows_per_block(H), down_rows_per_block(H, I));
        *err = b;
        return JitStatus::BadShape;
    }
    if (strncmp(arch, "gfx950", 6) != 0 || (arch[6] != '\0' && arch[6] != ':')) {
        *err = std::string("the kernels target gfx950 only, not ") + arch;
        return JitStatus::BadArch;
    }
    const bool chunk = chunk_shape_ok(H, I), lm = lm_head_shape_ok(H);
    const std::vector<KernelKey> keys = module_keys(H, I, chunk, lm);
    const std::string dir = (cache_dir != nullptr && cache_dir[0] != '\0') ? cache_dir : default_cache_dir();
    if (dir.empty()) {
        *err = "no cache directory: pass one, or set MOE_JIT_CACHE_DIR, XDG_CACHE_HOME or HOME";
        return JitStatus::CacheIo;
    }
    const uint64_t key = cache_key(H, I, "gfx950", chunk, lm);
    char fname[96];
    snprintf(fname, sizeof fname, "/moe_H%d_I%d_gfx950_%016llx.co", H, I, (unsigned long long)key);
    const std::string path = dir + fname;
    rep->chunk = chunk;
    rep->lm_head = lm;
    rep->kernels = (int)keys.size();
    snprintf(rep->file, sizeof rep->file, "%s", path.c_str());
    if (read_entry(path, key, keys, e)) {
        rep->from_cache = true;
        return JitStatus::Ok;
    }
    if (!make_dirs(dir, err)) return JitStatus::CacheIo;
    if (!compile(H, I, "gfx950", chunk, lm, keys, e, err)) return JitStatus::Compile;
    rep->from_cache = false;
    if (!write_entry(path, key, *e, err)) return JitStatus::CacheIo;
    return JitStatus::Ok;
}

double since(std::chrono::steady_clock::time_point t0)
{
    return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

bool kernel_expr(const KernelKey& k, char* buf, size_t n)
{
    const char* tf[2] = {"false", "true"};
    switch (k.kind) {
        case KernelKind::Quant: snprintf(buf, n, "moe::quant_kernel<%d>", k.H); return true;
        case KernelKind::Router: snprintf(buf, n, "moe::router_kernel<%d, %d>", k.H, k.v); return true;
        case KernelKind::GateUp: snprintf(buf, n, "moe::gate_up_kernel<%d, %d, %d>", k.H, k.I, k.v); return true;
        case KernelKind::Down:
            snprintf(buf, n, "moe::down_kernel<%d, %d, %d, %s>", k.H, k.I, k.v / 2, tf[k.v & 1]);
            return true;
        case KernelKind::Requant: snprintf(buf, n, "moe::requant_kernel<%d>", k.I); return true;
        case KernelKind::ChunkRouter: snprintf(buf, n, "moe::chunk_router_kernel<%d>", k.H); return true;
        case KernelKind::ChunkGateUp: snprintf(buf, n, "moe::chunk_gate_up_kernel<%d, %d>", k.H, k.I); return true;
        case KernelKind::ChunkDown:
            snprintf(buf, n, "moe::chunk_down_kernel<%d, %d, %s>", k.H, k.I, tf[k.v & 1]);
            return true;
        case KernelKind::Combine: snprintf(buf, n, "moe::combine_kernel<%d>", k.H); return true;
        case KernelKind::LmHead: snprintf(buf, n, "moe::lm_head_gemv_kernel<%d, %d>", k.H, k.v); return true;
        case KernelKind::Layer: snprintf(buf, n, "moe::layer_kernel<%d, %d, %d>", k.H, k.I, k.v); return true;
    }
    return false;
}

Kern find_kernel(const KernelKey& k)
{
    Kern out;
    if (g_n_mods.load(std::memory_order_acquire) == 0) {          // nothing loaded: compiled-in kernels only
        const AotKernel* a = aot_find(k);
        if (a != nullptr) out.aot = a->fn;
        return out;
    }
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return out;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_n_prefer.load(std::memory_order_relaxed) > 0 && (out.jit = module_find(k, device, true)) != nullptr)
        return out;
    if (const AotKernel* a = aot_find(k)) {
        out.aot = a->fn;
        return out;
    }
    out.jit = module_find(k, device, false);
    return out;
}

JitStatus jit_build(int H, int I, const char* arch, const char* cache_dir, JitReport* rep, std::string* err)
{
    const auto t0 = std::chrono::steady_clock::now();
    std::lock_guard<std::mutex> lock(g_mu);
    Entry e;
    const JitStatus st = get_entry(H, I, arch, cache_dir, &e, rep, err);
    rep->seconds = since(t0);
    return st;
}

JitStatus jit_load(int H, int I, const char* cache_dir, bool prefer, JitReport* rep, std::string* err)
{
    const auto t0 = std::chrono::steady_clock::now();
    int device = 0;
    hipError_t he = hipGetDevice(&device);
    hipDeviceProp_t prop;
    if (he == hipSuccess) he = hipGetDeviceProperties(&prop, device);
    if (he != hipSuccess) {
        *err = std::string("no HIP device: ") + hipGetErrorString(he);
        return JitStatus::Load;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Entry e;
    JitStatus st = get_entry(H, I, prop.gcnArchName, cache_dir, &e, rep, err);
    if (st != JitStatus::Ok) return st;
    auto* m = new LoadedModule{device, H, I, prefer, nullptr, e.keys, {}};
    he = hipModuleLoadData(&m->mod, e.code.data());
    for (size_t i = 0; he == hipSuccess && i < e.names.size(); ++i) {
        hipFunction_t f = nullptr;
        he = hipModuleGetFunction(&f, m->mod, e.names[i].c_str());
        m->fns.push_back(f);
    }
    if (he != hipSuccess) {
        if (m->mod != nullptr) hipModuleUnload(m->mod);
        delete m;
        *err = std::string("loading the compiled kernels failed: ") + hipGetErrorString(he);
        return JitStatus::Load;
    }
    // a shape loaded again on this device replaces its earlier module
    for (size_t i = 0; i < g_mods.size();) {
        LoadedModule* o = g_mods[i];
        if (o->device == device && o->H == H && o->I == I) {
            if (o->prefer) g_n_prefer.fetch_sub(1);
            hipModuleUnload(o->mod);
            delete o;
            g_mods.erase(g_mods.begin() + (long)i);
        } else {
            ++i;
        }
    }
    g_mods.push_back(m);
    if (prefer) g_n_prefer.fetch_add(1);
    g_n_mods.store((int)g_mods.size(), std::memory_order_release);
    rep->seconds = since(t0);
    return JitStatus::Ok;
}

int jit_unload(int H, int I)
{
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(g_mu);
    int n = 0;
    for (size_t i = 0; i < g_mods.size();) {
        LoadedModule* o = g_mods[i];
        if (o->device == device && o->H == H && o->I == I) {
            if (o->prefer) g_n_prefer.fetch_sub(1);
            hipModuleUnload(o->mod);
            delete o;
            g_mods.erase(g_mods.begin() + (long)i);
            ++n;
        } else {
            ++i;
        }
    }
    g_n_mods.store((int)g_mods.size(), std::memory_order_release);
    return n;
}

}  // namespace moe
