// Launch of the top-k gathered sparse MLA forward (kernels in fa_topk16.hip,
// part of the run-time loaded code object).
#include <stdio.h>

#include "fa_internal.h"

namespace fa {

hipError_t launch_topk(Dt dt, TopkParams& p, hipStream_t stream) {
  // One workgroup of 4 waves per (token, 128 query heads).
  p.n_htiles = (p.Hq + 127) / 128;
  const bool alias = p.v == p.k && p.v_ss == p.k_ss;
  char name[64];
  snprintf(name, sizeof(name), "fa_topk16_%s_v%d", dt == Dt::F16 ? "f16" : "bf16", alias ? 1 : 0);
  hipFunction_t fn = nullptr;
  hipError_t e = code_object_function(name, &fn);
  if (e != hipSuccess) return e;
  void* args[] = {&p};
  return hipModuleLaunchKernel(fn, (unsigned)(p.T * p.n_htiles), 1, 1, 256, 1, 1, 0, stream, args, nullptr);
}

}  // namespace fa
