// Caller-defined score_mods: run-time compilation (hipRTC) of the generic
// kernels of fa_custom.hpp around the caller's device functions, a cache of
// the loaded code objects per device and kernel configuration, and their
// launches.  The kernel sources are embedded in the library at build time
// (fa_rtc_sources.inc, generated from fa_common.hpp and fa_custom.hpp).
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/fa_mi355x.h"
#include "fa_rtc.hpp"

#include "fa_rtc_sources.inc"   // kRtcCommon, kRtcCustom, kRtcFwd32, kRtcBwd32

struct fa_score_mod_s {
  std::string source;
  std::mutex mu;
  struct Loaded {
    hipModule_t module;
    hipFunction_t fn[4];   // forward, query pass, key/value pass, forward over one key chunk
  };
  std::map<std::tuple<int, int, int, int, int, int>, Loaded> cache;   // device, dtype, D, causal, mask, block
};

namespace fa {
namespace {

const char* kKernelNames[4] = {"fa_custom_fwd", "fa_custom_dq", "fa_custom_dkdv", "fa_custom_fwd_split"};

// Kernels of a configuration: the forward, the two backward passes and the
// forward over one key chunk; fp32 at head_dim 512 has no key split.
int kernels_of(int dtype, int D) { return dtype == FA_F32 && D > 128 ? 3 : 4; }

// The translation unit: the caller's functions, then the kernel templates and
// one instantiation of each pass for the configuration (16-bit: the generic
// kernels of fa_custom.hpp; fp32: the library's fp32 kernels with MOD_CUSTOM).
std::string rtc_unit(const std::string& user, int dtype, int D, bool causal, bool mask, bool blk) {
  const char* tf[2] = {"false", "true"};
  const char* names[4] = {"fa_custom_fwd", "fa_custom_dq", "fa_custom_dkdv", "fa_custom_fwd_split"};
  std::string inst;
  char line[512];
  if (dtype == FA_F32) {
    inst = "\n#include \"fa_fwd32.hip\"\n#include \"fa_bwd32.hip\"\n";
    const char* bodies[4] = {"fwd32_body", "dq32_body", "dkdv32_body", "fwd32_body"};
    for (int i = 0; i < kernels_of(dtype, D); ++i) {
      snprintf(line, sizeof(line),
               "extern \"C\" __global__ __launch_bounds__(256, 1) void %s(const fa::AttnArgs a) "
               "{ fa::%s<%d, fa::MOD_CUSTOM, %s, %s, %s%s>(a); }\n",
               names[i], bodies[i], D, tf[causal], tf[mask], tf[blk], i == 3 ? ", true" : "");
      inst += line;
    }
    return user + "\n" + inst;
  }
  const char* T = dtype == FA_BF16 ? "fa::BF16" : "fa::F16";
  // workgroups per CU the registers allow: the forward fits two at either
  // head_dim (204 registers at 128), the backward passes at 128 one
  const int lb[4] = {2, D == 64 ? 2 : 1, D == 64 ? 2 : 1, 2};
  inst = "\n#include \"fa_custom.hpp\"\n";
  const char* bodies[4] = {"fwd_custom", "dq_custom", "dkdv_custom", "fwd_custom"};
  for (int i = 0; i < 4; ++i) {
    snprintf(line, sizeof(line),
             "extern \"C\" __global__ __launch_bounds__(256, %d) void %s(const fa::AttnArgs a) "
             "{ fa::%s<%s, %d, %s, %s, %s%s>(a); }\n",
             lb[i], names[i], bodies[i], T, D, tf[causal], tf[mask], tf[blk], i == 3 ? ", true" : "");
    inst += line;
  }
  return user + "\n" + inst;
}

// Compiles one configuration for `arch`; returns the code object or an
// empty vector with the compiler log in *log.
std::vector<char> rtc_compile(const std::string& unit, const std::string& arch, std::string* log) {
  hiprtcProgram prog;
  const char* headers[4] = {kRtcCommon, kRtcCustom, kRtcFwd32, kRtcBwd32};
  const char* names[4] = {"fa_common.hpp", "fa_custom.hpp", "fa_fwd32.hip", "fa_bwd32.hip"};
  if (hiprtcCreateProgram(&prog, unit.c_str(), "fa_score_mod.hip", 4, headers, names) != HIPRTC_SUCCESS) {
    *log = "hiprtcCreateProgram failed";
    return {};
  }
  const std::string arch_opt = "--offload-arch=" + arch;
  // no packed fp32 VALU instructions, as in the library's own build
  const char* opts[] = {arch_opt.c_str(), "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops",
#ifdef FA_DEBUG_BARRIERS
                        "-DFA_DEBUG_BARRIERS",   // the race-check library's kernels drain at every barrier
#endif
  };
  const hiprtcResult r = hiprtcCompileProgram(prog, (int)(sizeof(opts) / sizeof(opts[0])), opts);
  size_t n = 0;
  hiprtcGetProgramLogSize(prog, &n);
  log->assign(n, '\0');
  if (n) hiprtcGetProgramLog(prog, &(*log)[0]);
  std::vector<char> code;
  if (r == HIPRTC_SUCCESS) {
    size_t cs = 0;
    hiprtcGetCodeSize(prog, &cs);
    code.resize(cs);
    hiprtcGetCode(prog, code.data());
  }
  hiprtcDestroyProgram(&prog);
  return code;
}

std::string device_arch(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return "gfx950";
  std::string a = prop.gcnArchName;
  const size_t colon = a.find(':');
  return colon == std::string::npos ? a : a.substr(0, colon);
}

}  // namespace

fa_status custom_create(const char* source, fa_score_mod* out, char* log, size_t log_bytes) {
  if (!source || !out) return FA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  // one configuration compiled for the target, so that errors in the
  // caller's source surface here, with the compiler's log
  std::string msg;
  const std::vector<char> code = rtc_compile(rtc_unit(source, FA_F16, 64, false, false, false), "gfx950", &msg);
  if (log && log_bytes) {
    const size_t m = msg.size() < log_bytes - 1 ? msg.size() : log_bytes - 1;
    memcpy(log, msg.data(), m);
    log[m] = '\0';
  }
  if (code.empty()) return FA_ERR_COMPILE;
  fa_score_mod_s* s = new fa_score_mod_s;
  s->source = source;
  *out = s;
  return FA_OK;
}

fa_status custom_destroy(fa_score_mod mod) {
  if (!mod) return FA_ERR_INVALID_ARGUMENT;
  for (auto& kv : mod->cache) hipModuleUnload(kv.second.module);
  delete mod;
  return FA_OK;
}

fa_status custom_launch(fa_score_mod mod, int pass, int dtype, int D, bool causal, bool mask, bool blk,
                        const AttnArgs& a, unsigned grid, size_t shared_bytes, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  const auto key = std::make_tuple(dev, dtype, D, (int)causal, (int)mask, (int)blk);
  hipFunction_t fn;
  {
    std::lock_guard<std::mutex> lock(mod->mu);
    auto it = mod->cache.find(key);
    if (it == mod->cache.end()) {
      std::string log;
      const std::vector<char> code = rtc_compile(rtc_unit(mod->source, dtype, D, causal, mask, blk), device_arch(dev), &log);
      if (code.empty()) return FA_ERR_COMPILE;
      fa_score_mod_s::Loaded l;
      if (hipModuleLoadData(&l.module, code.data()) != hipSuccess) return FA_ERR_HIP;
      l.fn[3] = nullptr;
      for (int i = 0; i < kernels_of(dtype, D); ++i) {
        if (hipModuleGetFunction(&l.fn[i], l.module, kKernelNames[i]) != hipSuccess) {
          hipModuleUnload(l.module);
          return FA_ERR_HIP;
        }
      }
      it = mod->cache.emplace(key, l).first;
    }
    fn = it->second.fn[pass];
  }
  if (!fn) return FA_ERR_UNSUPPORTED;
  AttnArgs args = a;
  void* params[] = {&args};
  if (hipModuleLaunchKernel(fn, grid, 1, 1, 256, 1, 1, (unsigned)shared_bytes, st, params, nullptr) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

}  // namespace fa
