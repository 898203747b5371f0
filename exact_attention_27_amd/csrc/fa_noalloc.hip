// fa_backward_noalloc: the backward pass of fa_backward with its one workspace, the per-row
// delta vector D_i = rowsum(dO_i * O_i), held in a device array of fixed size that the library
// owns, so the call allocates nothing and takes no workspace argument. It is for callers that
// cannot allocate device memory: code under HIP graph capture, tight serving or training loops,
// harnesses that forbid allocation.
//
// The array lives for the life of the process, one copy per GPU (each device's code object
// holds its own). Its address on a device comes from hipGetSymbolAddress, taken once per device
// with that device current and cached; host code uses only that address (the array's name is a
// host-side stand-in, not a device address). Every call on one GPU shares the array: calls
// that overlap in time on one GPU (e.g. on two streams) race on it. The dQ kernel writes
// every D_i that it and the dK/dV kernel read before they read it, so nothing has to start at
// zero and no clearing is needed between calls.
#include <hip/hip_runtime.h>

#include <atomic>

#include "fa.h"

namespace {

// Rows of D the array holds: B*H*N may not exceed this (16 MiB of float32).
constexpr long long kNoAllocRows = 1LL << 22;

static __device__ __align__(256) float scratch[kNoAllocRows];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on that device.
// nullptr when the device index is out of range or the lookup fails.
float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
  // two threads racing here store the same address
  g_scratch_ptr[dev].store(static_cast<float*>(addr), std::memory_order_release);
  return static_cast<float*>(addr);
}

}  // namespace

extern "C" {

size_t fa_backward_noalloc_max_rows(void) { return (size_t)kNoAllocRows; }

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                        float scale, int dtype, void* stream) {
  // argument errors first, before any HIP call (fa_backward repeats every check)
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_INVALID_ARG;
  // B*H first, so the product with N cannot overflow
  if ((long long)B * H > kNoAllocRows || (long long)B * H * N > kNoAllocRows) return FA_ERR_UNSUPPORTED;
  float* delta = scratch_on_current_device();
  if (delta == nullptr) return FA_ERR_HIP;
  return fa_backward(q, k, v, o, dO, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, stream);
}

}  // extern "C"
