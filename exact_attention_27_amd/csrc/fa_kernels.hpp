// Internal launch interface between the C ABI (fa_api.cpp) and the kernel translation units.
// Arguments here are already validated; sizes fit the kernels' index arithmetic.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace fa {

// Element strides of one (B, H, N, d) operand: element (b, h, r, c) sits at
// base + b*b + h*h + r*r + c (the d elements of a row are contiguous). With variable-length
// sequences the batch stride is unused: row r of sequence b is row cu[b] + r of the packed
// operand.
struct Strides {
  long long b, h, r;
};

// Problem geometry. Query-side operands (Q, O, dO, dQ; LSE, delta) and key-side operands
// (K, V, dK, dV) may have different lengths. Fixed length (cu == nullptr): every sequence
// has N query rows and Nk key rows, and LSE / delta are (B, H, N) contiguous. Variable
// length: sequence b is query rows [cu[b], cu[b+1]) and key rows [cuk[b], cuk[b+1]) of the
// packed operands (T and Tk rows in all), N and Nk bound the lengths, and LSE / delta are
// (H, T) contiguous. A workgroup clamps what it reads from cu / cuk to [0, T] / [0, Tk] and
// the lengths to N / Nk, so no contents of them lead it outside the operands. With the causal
// mask the queries are the last positions of their sequence: query i sees key j iff
// j <= i + (nk - n).
struct Geom {
  int B, H, N;
  const int* cu;
  int T;
  int dh;  // head dim of the operands: a multiple of 8, at most the kernel's D; the columns
           // [dh, D) of every tile are zero on chip and never stored
  int Nk;
  const int* cuk;
  int Tk;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  Strides sq, sk, sv, so;
  Geom g;
  int d;
  bool causal, bf16;
  float c_log2;  // scale * log2(e)
  void* stream;
  int splits = 0;         // > 0: split-KV forward with this many key ranges per Q tile
  float* part = nullptr;  // split-KV partial states (see fwd_kernel), splits > 0 only
  bool pingpong = false;  // the two-group ping-pong schedule (128-wide tiles, splits == 0)
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
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  Geom g;
  int d;
  bool causal, bf16;
  float scale;
  float c_log2;
  void* stream;
  bool dq_delta = false;  // the dQ stage computes D from o and dO and writes it to delta
};

// Launch `kern` and return the status of this launch alone. hipLaunchKernel reports the
// launch's own outcome, where hipGetLastError() after a <<<>>> launch would also return an
// error left pending on the thread by some earlier, unrelated HIP call. The arguments are
// converted to the kernel's parameter types first and passed by address.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kern)(KArgs...), unsigned grid, unsigned block, void* stream,
                                Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count must match the kernel's");
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(block), ptrs, 0,
                         static_cast<hipStream_t>(stream));
}

// Causal grids pair a heavy and a light tile per workgroup, so that every workgroup has the
// same work, when the paired grid still gives every CU at least two workgroups; smaller grids
// run one tile per workgroup, heaviest first, which shortens the longest workgroup.
bool pair_causal_tiles(long long paired_grid);

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_dkv(const BwdArgs& a);
hipError_t launch_bwd_dkv_wide(const BwdArgs& a);  // head dims above 128 (its own unit)
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace fa
