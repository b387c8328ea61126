// Run-time loading of the code object that holds the 16-bit forward kernels
// (built from fa_fwd16.hip and fa_topk16.hip by build.py and embedded here as
// a byte array) and lookup of its kernels by name, once per device.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "fa_internal.h"
#include "fa_kernels_hsaco.inc"

namespace fa {
namespace {

struct DeviceModule {
  hipModule_t module = nullptr;
  std::unordered_map<std::string, hipFunction_t> functions;
};

std::mutex g_mutex;
std::vector<DeviceModule> g_modules;

}  // namespace

hipError_t code_object_function(const char* name, hipFunction_t* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mutex);
  if ((int)g_modules.size() <= dev) g_modules.resize(dev + 1);
  DeviceModule& dm = g_modules[dev];
  if (!dm.module) {
    e = hipModuleLoadData(&dm.module, kCodeObject);
    if (e != hipSuccess) {
      dm.module = nullptr;
      return e;
    }
  }
  auto it = dm.functions.find(name);
  if (it != dm.functions.end()) {
    *fn = it->second;
    return hipSuccess;
  }
  hipFunction_t f = nullptr;
  e = hipModuleGetFunction(&f, dm.module, name);
  if (e != hipSuccess) return e;
  dm.functions.emplace(name, f);
  *fn = f;
  return hipSuccess;
}

}  // namespace fa
