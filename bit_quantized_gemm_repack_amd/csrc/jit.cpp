// Run-time specialisation of the dense GEMM kernels: hipRTC compile, code
// object cache (memory per device, disk per key), module launch.  See jit.h.
#include "jit.h"

#include <dlfcn.h>
#include <hip/hip_ext.h>
#include <hip/hiprtc.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <cerrno>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

namespace hq::jit {
namespace {

constexpr const char* kMagic = "HQJIT1\n";  // code-object file: magic, lowered name, '\n', code

// Kernel headers a specialisation's source may include (the source hash covers
// all of them, so an edited kernel never loads a stale code object).
const char* const kSources[] = {"device_common.h", "hq_internal.h", "qgemm_skinny_kernel.h", "qgemm_tiled_kernel.h"};

std::mutex g_mu;
std::unordered_map<std::string, hipFunction_t> g_funcs;  // "device:key" -> kernel
std::atomic<int64_t> g_compiles{0}, g_disk_hits{0}, g_memory_hits{0}, g_launches{0};
double g_compile_s = 0.0, g_load_s = 0.0;  // under g_mu

uint64_t fnv1a(const void* data, size_t n, uint64_t h = 1469598103934665603ull) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

// <package>/csrc: the kernel sources sit next to the loaded library.
const std::string& source_dir() {
  static const std::string dir = [] {
    Dl_info info{};
    std::string lib = dladdr(reinterpret_cast<void*>(&fnv1a), &info) && info.dli_fname ? info.dli_fname : "";
    const size_t slash = lib.rfind('/');
    return (slash == std::string::npos ? std::string(".") : lib.substr(0, slash)) + "/csrc";
  }();
  return dir;
}

bool read_file(const std::string& path, std::string* out) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  std::fseek(f, 0, SEEK_END);
  const long n = std::ftell(f);
  std::fseek(f, 0, SEEK_SET);
  out->resize(n > 0 ? (size_t)n : 0);
  const size_t got = n > 0 ? std::fread(&(*out)[0], 1, (size_t)n, f) : 0;
  std::fclose(f);
  return got == out->size();
}

// Hash of the kernel sources (0 if one cannot be read: then every key says so
// and no cache file can match a readable build).
uint64_t sources_hash() {
  static const uint64_t h = [] {
    uint64_t v = 1469598103934665603ull;
    for (const char* name : kSources) {
      std::string text;
      if (!read_file(source_dir() + "/" + name, &text)) return uint64_t(0);
      v = fnv1a(name, std::strlen(name), v);
      v = fnv1a(text.data(), text.size(), v);
    }
    return v;
  }();
  return h;
}

// Only options every hipRTC accepts: the compiler is whichever hipRTC the
// process loaded (a framework may bring its own ROCm), and an option its LLVM
// does not know ends the process.  So no -mllvm options: the run-time
// kernels keep the compiler's default register form for matrix results.
std::vector<std::string> options(const Spec&, const std::string& arch) {
  return {"--offload-arch=" + arch, "-O3", "-std=c++20", "-I" + source_dir(),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
}

bool mkdirs(const std::string& dir) {
  std::string cur;
  for (size_t i = 0; i <= dir.size(); ++i) {
    if (i == dir.size() || dir[i] == '/') {
      if (!cur.empty() && ::mkdir(cur.c_str(), 0755) != 0 && errno != EEXIST) return false;
    }
    if (i < dir.size()) cur.push_back(dir[i]);
  }
  return true;
}

std::string cache_dir(const hq_plan* p) {
  if (p->jit_dir[0]) return p->jit_dir;
  if (const char* e = std::getenv("HQ_JIT_CACHE_DIR"); e && *e) return e;
  if (const char* x = std::getenv("XDG_CACHE_HOME"); x && *x) return std::string(x) + "/hq_jit";
  if (const char* h = std::getenv("HOME"); h && *h) return std::string(h) + "/.cache/hq_jit";
  return "/tmp/hq_jit";
}

std::string device_arch(int dev) {
  hipDeviceProp_t prop{};
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return "";
  std::string a = prop.gcnArchName;
  const size_t colon = a.find(':');
  return colon == std::string::npos ? a : a.substr(0, colon);
}

// hipRTC compile of one specialisation: lowered kernel name and code object.
bool compile(const Spec& s, const std::string& arch, std::string* lowered, std::string* code, std::string* log) {
  const std::string src = "#include \"" + s.header + "\"\n";
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, src.c_str(), "hq_jit.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS) {
    *log = "hiprtcCreateProgram failed";
    return false;
  }
  hiprtcAddNameExpression(prog, s.expr.c_str());
  const std::vector<std::string> opts = options(s, arch);
  std::vector<const char*> o;
  for (const std::string& x : opts) o.push_back(x.c_str());
  const hiprtcResult r = hiprtcCompileProgram(prog, (int)o.size(), o.data());
  bool ok = r == HIPRTC_SUCCESS;
  if (!ok) {
    size_t n = 0;
    hiprtcGetProgramLogSize(prog, &n);
    std::string text(n, '\0');
    if (n) hiprtcGetProgramLog(prog, &text[0]);
    *log = std::string(hiprtcGetErrorString(r)) + ": " + text.substr(0, 2000);
  } else {
    const char* name = nullptr;
    size_t n = 0;
    ok = hiprtcGetLoweredName(prog, s.expr.c_str(), &name) == HIPRTC_SUCCESS && name &&
         hiprtcGetCodeSize(prog, &n) == HIPRTC_SUCCESS && n > 0;
    if (ok) {
      *lowered = name;
      code->assign(n, '\0');
      ok = hiprtcGetCode(prog, &(*code)[0]) == HIPRTC_SUCCESS;
    }
    if (!ok) *log = "hipRTC produced no code object";
  }
  hiprtcDestroyProgram(&prog);
  return ok;
}

// The cache file: magic, lowered name, '\n', code object.  Written under a
// temporary name and renamed, so a reader never sees a partial file.
bool load_cached(const std::string& path, std::string* lowered, std::string* code) {
  std::string data;
  if (!read_file(path, &data)) return false;
  const size_t m = std::strlen(kMagic);
  if (data.compare(0, m, kMagic) != 0) return false;
  const size_t nl = data.find('\n', m);
  if (nl == std::string::npos || nl + 1 >= data.size()) return false;
  *lowered = data.substr(m, nl - m);
  *code = data.substr(nl + 1);
  return true;
}

void store_cached(const std::string& dir, const std::string& path, const std::string& lowered,
                  const std::string& code) {
  if (!mkdirs(dir)) return;  // no cache: the next process compiles again
  const std::string tmp = path + ".tmp." + std::to_string((long)::getpid());
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) return;
  bool ok = std::fwrite(kMagic, 1, std::strlen(kMagic), f) == std::strlen(kMagic) &&
            std::fwrite(lowered.data(), 1, lowered.size(), f) == lowered.size() && std::fputc('\n', f) != EOF &&
            std::fwrite(code.data(), 1, code.size(), f) == code.size();
  ok = (std::fclose(f) == 0) && ok;
  if (!ok || std::rename(tmp.c_str(), path.c_str()) != 0) std::remove(tmp.c_str());
}

// The kernel of a specialisation on the current device: memory, else disk,
// else compile (and store).
int get_function(const hq_plan* p, const Spec& s, hipFunction_t* fn, std::string* err_msg) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  const std::string arch = device_arch(dev);
  if (arch.empty()) return (int)hipErrorInvalidDevice;
  const std::string key = cache_key(s, arch);
  const std::string mkey = std::to_string(dev) + ":" + key;
  std::lock_guard<std::mutex> lock(g_mu);
  if (auto it = g_funcs.find(mkey); it != g_funcs.end()) {
    ++g_memory_hits;
    *fn = it->second;
    return hipSuccess;
  }
  const std::string dir = cache_dir(p);
  const std::string path = dir + "/" + key + ".co";
  std::string lowered, code;
  const auto t0 = std::chrono::steady_clock::now();
  if (load_cached(path, &lowered, &code)) {
    ++g_disk_hits;
  } else {
    std::string log;
    if (!compile(s, arch, &lowered, &code, &log)) {
      if (err_msg) *err_msg = "run-time compile of " + s.expr + " failed: " + log;
      return (int)hipErrorInvalidImage;
    }
    ++g_compiles;
    g_compile_s += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    store_cached(dir, path, lowered, code);
  }
  const auto t1 = std::chrono::steady_clock::now();
  hipModule_t mod = nullptr;
  e = hipModuleLoadData(&mod, code.data());
  if (e == hipSuccess) e = hipModuleGetFunction(fn, mod, lowered.c_str());
  if (e != hipSuccess) {
    if (err_msg) *err_msg = "loading the code object of " + s.expr + ": " + hipGetErrorString(e);
    return (int)e;
  }
  g_load_s += std::chrono::duration<double>(std::chrono::steady_clock::now() - t1).count();
  g_funcs.emplace(mkey, *fn);  // modules stay loaded until the process ends
  return hipSuccess;
}

}  // namespace

int prepare(const hq_plan* p, const Spec& s, const std::string& arch, std::string* err_msg) {
  const std::string key = cache_key(s, arch);
  const std::string dir = cache_dir(p);
  const std::string path = dir + "/" + key + ".co";
  std::lock_guard<std::mutex> lock(g_mu);
  std::string lowered, code;
  if (load_cached(path, &lowered, &code)) {
    ++g_disk_hits;
    return 0;
  }
  std::string log;
  const auto t0 = std::chrono::steady_clock::now();
  if (!compile(s, arch, &lowered, &code, &log)) {
    if (err_msg) *err_msg = "run-time compile of " + s.expr + " failed: " + log;
    return 1;
  }
  ++g_compiles;
  g_compile_s += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  store_cached(dir, path, lowered, code);
  if (!load_cached(path, &lowered, &code)) {
    if (err_msg) *err_msg = "cannot write the code-object cache file " + path;
    return 2;
  }
  return 0;
}

namespace {

template <typename Args>
int launch(hipFunction_t fn, dim3 grid, dim3 block, const Args& a, void* stream) {
  Args copy = a;
  void* params[] = {&copy};
  const TimingEvents ev = take_timing();
  ++g_launches;
  return (int)hipExtModuleLaunchKernel(fn, grid.x * block.x, grid.y * block.y, grid.z * block.z, block.x, block.y,
                                       block.z, 0, static_cast<hipStream_t>(stream), params, nullptr,
                                       static_cast<hipEvent_t>(ev.start), static_cast<hipEvent_t>(ev.stop), 0);
}


}  // namespace

Spec skinny_spec(int fmt, const SkinnyCfg& cfg, int64_t m, int64_t n, int64_t k) {
  const int maxt = cfg.waves > 8 ? 1024 : 512;
  const int stages = cfg.stages > 0 ? cfg.stages : 2;
  char buf[160];
  std::snprintf(buf, sizeof(buf), "hq::qgemm_skinny<%d,%d,%d,%d,%d,0,%lld,%lld,%lld,1>", fmt, cfg.mb, cfg.nb, stages,
                maxt, (long long)m, (long long)n, (long long)k);
  return Spec{"qgemm_skinny_kernel.h", buf};
}

Spec tiled_spec(int fmt, const TiledCfgRt& cfg, int64_t m, int64_t n, int64_t k) {
  char buf[160];
  std::snprintf(buf, sizeof(buf), "hq::qgemm_tiled<%d,%d,%d,0,%d,%lld,%lld,%lld,1>", fmt, cfg.bm, cfg.nbw,
                cfg.stages > 0 ? cfg.stages : 3, (long long)m, (long long)n, (long long)k);
  return Spec{"qgemm_tiled_kernel.h", buf};
}

std::string cache_key(const Spec& s, const std::string& arch) {
  uint64_t h = sources_hash();
  int major = 0, minor = 0;
  hiprtcVersion(&major, &minor);  // the compiler that would build it
  h = fnv1a(&major, sizeof(major), h);
  h = fnv1a(&minor, sizeof(minor), h);
  const std::string text = s.header + "|" + s.expr + "|" + arch;
  h = fnv1a(text.data(), text.size(), h);
  for (const std::string& o : options(s, arch)) {
    if (o.rfind("-I", 0) == 0) continue;  // where the sources sit does not change the code
    h = fnv1a(o.data(), o.size(), h);
  }
  const char* kind = s.header.find("skinny") != std::string::npos ? "skinny" : "tiled";
  char buf[96];
  std::snprintf(buf, sizeof(buf), "hq-%s-%s-%016llx", kind, arch.c_str(), (unsigned long long)h);
  return buf;
}

int launch_skinny(const hq_plan* p, const SkinnyCfg& cfg, const SkinnyArgs& a, void* stream, std::string* err_msg) {
  // every split holds at least one group, and the splits cover K (as the precompiled launcher)
  if (a.G < 1 || a.gps < 1 || (int64_t)(cfg.split - 1) * a.gps >= a.G || (int64_t)cfg.split * a.gps < a.G ||
      cfg.waves < 1 || cfg.waves > 16 || (cfg.waves > 8 && (cfg.mb != 1 || cfg.nb != 1)))
    return (int)hipErrorInvalidValue;
  hipFunction_t fn = nullptr;
  const int e = get_function(p, skinny_spec(p->fmt, cfg, a.M, a.N, a.K), &fn, err_msg);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(a.N / (16 * cfg.nb)), (unsigned)cfg.split, (unsigned)((a.M + 16 * cfg.mb - 1) / (16 * cfg.mb)));
  return launch(fn, grid, dim3(64 * cfg.waves), a, stream);
}

int launch_tiled(const hq_plan* p, const TiledCfgRt& cfg, const TiledArgs& a, void* stream, std::string* err_msg) {
  const int split = a.part ? cfg.split : 1;
  if (a.G < 1 || a.gps < 1 || (int64_t)(split - 1) * a.gps >= a.G || (int64_t)split * a.gps < a.G)
    return (int)hipErrorInvalidValue;
  hipFunction_t fn = nullptr;
  const int e = get_function(p, tiled_spec(p->fmt, cfg, a.M, a.N, a.K), &fn, err_msg);
  if (e != hipSuccess) return e;
  return launch(fn, dim3((unsigned)(a.tiles_m * a.tiles_n), (unsigned)split), dim3(256), a, stream);
}

Stats stats() {
  std::lock_guard<std::mutex> lock(g_mu);
  return Stats{g_compiles.load(), g_disk_hits.load(), g_memory_hits.load(), g_launches.load(), g_compile_s, g_load_s};
}

}  // namespace hq::jit
