// Internal launch interface between the C ABI (fa_api.cpp) and the kernel translation units.
// Arguments here are already validated; sizes fit the kernels' index arithmetic.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int BH, N, d;
  bool causal, bf16;
  float c_log2;  // scale * log2(e)
  void* stream;
  int splits = 0;         // > 0: split-KV forward with this many key ranges per Q tile
  float* part = nullptr;  // split-KV partial states (see fwd_kernel), splits > 0 only
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int BH, N, d;
  bool causal, bf16;
  float scale;
  float c_log2;
  void* stream;
};

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_dkv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace fa
