// Internal launcher interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;
  int n_qtiles;      // filled in by the launcher
  float scale_log2;  // softmax scale * log2(e)
};

// Enqueue the 16-bit forward.  Arguments are validated by the caller.
hipError_t launch_fwd(const FwdArgs& a, int B, int H, int d, int dtype, bool causal,
                      hipStream_t stream);

}  // namespace fa
