// C ABI of libfa.so: host-side validation and kernel dispatch. Declarations and the full
// contract (layouts, ownership, streams, errors) are in include/fa.h.
//
// Every check runs on the host before anything is enqueued; a request the kernels do not
// implement is refused with FA_ERR_UNSUPPORTED rather than served by a slower or
// approximate path (an unnoticed backend fallback is the failure mode warned about in
// "FlashAttentionを1から", section "現場ではこう使う").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_kernels.hpp"

namespace {

constexpr double kLog2eD = 1.4426950408889634;

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common shape/type/scale validation. On success, fills `elems` = B*H*N*d, `rows` = B*H*N.
int check_common(int B, int H, int N, int d, int causal, float scale, int dtype, long long* elems,
                 long long* rows) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_FP16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  // 64-bit overflow of the element count (and of its byte size), and the kernels' grid
  // arithmetic, which indexes heads with 32-bit ints.
  const long long bh = (long long)B * (long long)H;
  if (bh > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  const long long r = bh * (long long)N;
  if (r / N != bh) return FA_ERR_INVALID_ARG;
  const long long e = r * (long long)d;
  if (e / d != r || e > (0x7fffffffffffffffLL / 4)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (N > (1 << 30)) return FA_ERR_UNSUPPORTED;
  // Grid size: (N / 64) * B*H workgroups must fit a 32-bit grid dimension.
  const long long tiles = ((long long)N + 63) / 64;
  if (tiles * bh > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  *elems = e;
  *rows = r;
  return FA_OK;
}

Span span(const void* p, long long bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, lo + (uintptr_t)bytes};
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK:
      return "FA_OK";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: valid request not implemented by this library";
    case FA_ERR_HIP:
      return "FA_ERR_HIP: HIP runtime reported an error";
    default:
      return "unknown fa_status";
  }
}

}  // extern "C"

namespace {

// Most key ranges one Q tile may be cut into.
constexpr int kMaxSplits = 256;

// Bytes of split-KV workspace: per split and row, d fp32 accumulators, a max and a sum.
long long splitkv_bytes(long long rows, int d, int splits) { return (long long)splits * rows * (d + 2) * 4; }

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                 int causal, float scale, int dtype, int splits, float* part, size_t part_bytes, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return FA_ERR_INVALID_ARG;
  long long elems = 0, rows = 0;
  const int st = check_common(B, H, N, d, causal, scale, dtype, &elems, &rows);
  if (st != FA_OK) return st;
  const long long tb = elems * 2;
  const Span sq = span(q, tb), sk = span(k, tb), sv = span(v, tb), so = span(o, tb);
  if (overlaps(so, sq) || overlaps(so, sk) || overlaps(so, sv)) return FA_ERR_INVALID_ARG;
  if (lse) {
    const Span sl = span(lse, rows * 4);
    if (overlaps(sl, sq) || overlaps(sl, sk) || overlaps(sl, sv) || overlaps(sl, so)) return FA_ERR_INVALID_ARG;
  }
  if (splits > 0) {
    if (!part || !aligned16(part)) return FA_ERR_INVALID_ARG;
    const long long need = splitkv_bytes(rows, d, splits);
    if ((unsigned long long)need > (unsigned long long)part_bytes) return FA_ERR_INVALID_ARG;
    const Span sp = span(part, need);
    if (overlaps(sp, sq) || overlaps(sp, sk) || overlaps(sp, sv) || overlaps(sp, so)) return FA_ERR_INVALID_ARG;
    if (lse && overlaps(sp, span(lse, rows * 4))) return FA_ERR_INVALID_ARG;
    // grid = (N / 128 Q tiles) * splits * B*H workgroups in one 32-bit grid dimension
    if (((long long)N + 127) / 128 * splits * ((long long)B * H) > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  }
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.N = N;
  a.d = d;
  a.causal = causal != 0;
  a.bf16 = dtype == FA_BF16;
  a.c_log2 = (float)((double)scale * kLog2eD);
  a.stream = stream;
  a.splits = splits;
  a.part = part;
  return fa::launch_forward(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, 0, nullptr, 0, stream);
}

size_t fa_forward_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  if (num_splits < 1 || num_splits > kMaxSplits) return 0;
  long long elems = 0, rows = 0;
  if (check_common(B, H, N, d, 0, 1.0f, FA_BF16, &elems, &rows) != FA_OK) return 0;
  return (size_t)splitkv_bytes(rows, d, num_splits);
}

int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       int d, int causal, float scale, int dtype, int num_splits, float* workspace,
                       size_t workspace_bytes, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, num_splits, workspace, workspace_bytes,
                      stream);
}

// Shared validation of backward arguments. Null entries are arguments a stage does not use.
static int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                     const void* dq, const void* dk, const void* dv, const float* delta, int B, int H, int N,
                     int d, int causal, float scale, int dtype, bool need_qkv, bool need_o, bool need_dq,
                     bool need_dkv, fa::BwdArgs* a) {
  if (!dO || !delta) return FA_ERR_INVALID_ARG;
  if (need_qkv && (!q || !k || !v || !lse)) return FA_ERR_INVALID_ARG;
  if (need_o && !o) return FA_ERR_INVALID_ARG;
  if (need_dq && !dq) return FA_ERR_INVALID_ARG;
  if (need_dkv && (!dk || !dv)) return FA_ERR_INVALID_ARG;
  const void* all[] = {q, k, v, o, dO, lse, dq, dk, dv, delta};
  for (const void* p : all)
    if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
  long long elems = 0, rows = 0;
  const int st = check_common(B, H, N, d, causal, scale, dtype, &elems, &rows);
  if (st != FA_OK) return st;
  const long long tb = elems * 2, fb = rows * 4;
  // inputs of this call; `delta` is an input of the dK/dV and dQ stages, an output of the
  // preprocess stage
  const bool delta_out = need_o;
  Span ins[7];
  int nin = 0;
  const void* in_t[] = {q, k, v, o, dO};
  for (const void* p : in_t)
    if (p) ins[nin++] = span(p, tb);
  if (lse) ins[nin++] = span(lse, fb);
  if (!delta_out) ins[nin++] = span(delta, fb);
  Span outs[4];
  int nout = 0;
  if (dq) outs[nout++] = span(dq, tb);
  if (dk) outs[nout++] = span(dk, tb);
  if (dv) outs[nout++] = span(dv, tb);
  if (delta_out) outs[nout++] = span(delta, fb);
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
  }
  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->dO = dO;
  a->lse = lse;
  a->dq = const_cast<void*>(dq);
  a->dk = const_cast<void*>(dk);
  a->dv = const_cast<void*>(dv);
  a->delta = const_cast<float*>(delta);
  a->BH = B * H;
  a->N = N;
  a->d = d;
  a->causal = causal != 0;
  a->bf16 = dtype == FA_BF16;
  a->scale = scale;
  a->c_log2 = (float)((double)scale * kLog2eD);
  return FA_OK;
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, int causal, float scale,
                int dtype, void* stream) {
  fa::BwdArgs a;
  // delta is written by the first stage and read by the other two: validate it as an output.
  int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, true, true, true,
                     true, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  if (fa::launch_bwd_preprocess(a) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_dkv(a) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_dq(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_backward_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d, int dtype,
                           void* stream) {
  fa::BwdArgs a;
  // the preprocess stage ignores causal and scale; validate them at neutral values
  int st = check_bwd(nullptr, nullptr, nullptr, o, dO, nullptr, nullptr, nullptr, nullptr, delta, B, H, N, d, 0,
                     1.0f, dtype, false, true, false, false, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  return fa::launch_bwd_preprocess(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dkv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                    const float* delta, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                    int dtype, void* stream) {
  fa::BwdArgs a;
  int st = check_bwd(q, k, v, nullptr, dO, lse, nullptr, dk, dv, delta, B, H, N, d, causal, scale, dtype, true,
                     false, false, true, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  return fa::launch_bwd_dkv(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                   const float* delta, void* dq, int B, int H, int N, int d, int causal, float scale, int dtype,
                   void* stream) {
  fa::BwdArgs a;
  int st = check_bwd(q, k, v, nullptr, dO, lse, dq, nullptr, nullptr, delta, B, H, N, d, causal, scale, dtype,
                     true, false, true, false, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
