// Run-time specialisation of the dense GEMM kernels (hq_plan_set_jit).
//
// The pages compile each layer's kernel at run time with the layer's shape
// fixed and keep the compiled kernels in a cache ("Humming: open-source
// kernel library for quantized inference", news.ditty.ir, summary: compile
// time of one kernel brought from 23.35 s to 1.82 s; news.cocoloop.cn,
// limitations section, compile-speed paragraph: about 1.9 s per kernel and a
// few seconds of warm-up per layer).  Here the same kernel templates the
// library ships precompiled are compiled by hipRTC for gfx950 with the call's
// M, N and K as template constants (plus the format and the execution choice
// the heuristic or the tuning table picked), and the code object is kept in
// memory per device and on disk per key.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "hq_internal.h"

namespace hq::jit {

// One specialised kernel: the template expression hipRTC instantiates and the
// compile options it is built with.
struct Spec {
  std::string header;  // kernel header the source includes
  std::string expr;    // e.g. "hq::qgemm_skinny<1,1,1,2,512,0,1,4096,4096,1>"
};

// The specialisation of the skinny / tiled kernel for one dense call.
Spec skinny_spec(int fmt, const SkinnyCfg& cfg, int64_t m, int64_t n, int64_t k);
Spec tiled_spec(int fmt, const TiledCfgRt& cfg, int64_t m, int64_t n, int64_t k);

// Cache key of a specialisation for an architecture (e.g. "gfx950"): a
// readable prefix and a 64-bit hash of the key fields, the kernel sources,
// the compile options and the hipRTC version; the code object's file name is
// key + ".co".
std::string cache_key(const Spec& s, const std::string& arch);

// Compile a specialisation for `arch` into the plan's cache directory unless
// a valid code object is there already (no device needed): 0 on success, the
// reason in err_msg otherwise.
int prepare(const hq_plan* p, const Spec& s, const std::string& arch, std::string* err_msg);

// Launches of a specialisation (compiled or loaded on first use per device);
// a hipError_t as int, with the compile log kept for hq_last_error on a
// failed compile (err_msg).
int launch_skinny(const hq_plan* p, const SkinnyCfg& cfg, const SkinnyArgs& a, void* stream, std::string* err_msg);
int launch_tiled(const hq_plan* p, const TiledCfgRt& cfg, const TiledArgs& a, void* stream, std::string* err_msg);

// Counters since load (hq_jit_get_stats).
struct Stats {
  int64_t compiles, disk_hits, memory_hits, launches;
  double compile_seconds, load_seconds;
};
Stats stats();

}  // namespace hq::jit
