// C ABI of libfa.so: host-side validation and kernel dispatch. Declarations and the full
// contract (layouts, ownership, streams, errors) are in include/fa.h.
//
// Every check runs on the host before anything is enqueued; a request the kernels do not
// implement is refused with FA_ERR_UNSUPPORTED rather than served by a slower or
// approximate path (an unnoticed backend fallback is the failure mode warned about in
// "FlashAttentionを1から", section "現場ではこう使う").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_kernels.hpp"

namespace {

constexpr double kLog2eD = 1.4426950408889634;
// Row strides up to 2^23 elements keep every source offset inside a 128-row tile below 2^31
// bytes, under the kernels' out-of-range offset (2^31) used to zero the columns past d. (The
// 256-wide kernels stage tiles of at most 128 rows too.)
constexpr long long kMaxRowStride = 1LL << 23;
constexpr long long kMaxExtent = 1LL << 60;     // elements an operand may span

using u128 = unsigned __int128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One dimension of an operand's address map: `count` indices `stride` elements apart.
struct Dim {
  long long stride, count;
};

// A 16-bit operand (element size 2) or a float32 statistics array (contiguous rows).
struct Operand {
  uintptr_t base = 0;
  Dim dims[4];  // row elements, head, row, batch (batch unused with variable lengths)
  int ndims = 0;
  long long extent = 0;  // elements from base to one past the last one addressed
  int esize = 2;
  bool has_strides = false;
  fa::Strides st{};
};

// Key-side length bound, offsets and row count of a problem (defaults: the query side's).
int nk_of(const fa_problem& p) { return p.N_k > 0 ? p.N_k : p.N; }
const int* cuk_of(const fa_problem& p) { return p.cu_seqlens_k ? p.cu_seqlens_k : p.cu_seqlens; }
int totalk_of(const fa_problem& p) { return p.cu_seqlens_k ? p.total_k : p.total; }
// Rows of a query-side / key-side operand.
long long qrows(const fa_problem& p) { return p.cu_seqlens ? p.total : p.N; }
long long krows(const fa_problem& p) { return p.cu_seqlens ? totalk_of(p) : nk_of(p); }

// Shape checks shared by every entry point.
int check_shape(const fa_problem& p) {
  if (p.B <= 0 || p.H <= 0 || p.d <= 0 || p.N <= 0 || p.N_k < 0) return FA_ERR_INVALID_ARG;
  if (p.dtype != FA_FP16 && p.dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (p.causal != 0 && p.causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(p.scale) || !(p.scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (p.cu_seqlens != nullptr && (p.total < 0 || !aligned16(p.cu_seqlens))) return FA_ERR_INVALID_ARG;
  if (p.cu_seqlens_k != nullptr && (p.cu_seqlens == nullptr || p.total_k < 0 || !aligned16(p.cu_seqlens_k)))
    return FA_ERR_INVALID_ARG;
  const long long bh = (long long)p.B * p.H;
  if (bh > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  // head dims: multiples of 8 up to 256, run on the 64-, 128- or 256-wide kernels with the
  // columns past d zero on chip
  if (p.d % 8 != 0 || p.d > 256) return FA_ERR_UNSUPPORTED;
  if (p.N > (1 << 30) || nk_of(p) > (1 << 30)) return FA_ERR_UNSUPPORTED;
  // Grids: (N / 64) * B*H and (N_k / 64) * B*H tile workgroups, and (statistics rows / 4) *
  // heads row blocks, in one 32-bit grid dimension.
  if (((long long)p.N + 63) / 64 * bh > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  if (((long long)nk_of(p) + 63) / 64 * bh > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  const long long stat = p.cu_seqlens ? (long long)p.H * p.total : bh * p.N;
  if (stat / 4 + bh > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// A 16-bit operand of the problem with strides s and `rows` rows per head (qrows or krows);
// FA_OK or FA_ERR_INVALID_ARG.
int make_operand(const fa_problem& p, const void* data, const fa_strides& s, long long rows, Operand* op) {
  if (!data || !aligned16(data)) return FA_ERR_INVALID_ARG;
  const bool varlen = p.cu_seqlens != nullptr;
  const long long sb = varlen ? 0 : s.batch;
  if (sb < 0 || s.head < 0 || s.row < p.d || s.row > kMaxRowStride) return FA_ERR_INVALID_ARG;
  if ((sb | s.head | s.row) & 7) return FA_ERR_INVALID_ARG;
  op->base = reinterpret_cast<uintptr_t>(data);
  op->ndims = 0;
  op->dims[op->ndims++] = Dim{1, p.d};
  op->dims[op->ndims++] = Dim{s.head, p.H};
  op->dims[op->ndims++] = Dim{s.row, rows};
  if (!varlen) op->dims[op->ndims++] = Dim{sb, p.B};
  u128 last = 0;
  for (int i = 0; i < op->ndims; ++i)
    if (op->dims[i].count > 0) last += (u128)(op->dims[i].count - 1) * (u128)op->dims[i].stride;
  if (rows == 0) last = 0;
  if (last >= (u128)kMaxExtent) return FA_ERR_INVALID_ARG;
  op->extent = rows == 0 ? 0 : (long long)last + 1;
  op->esize = 2;
  op->has_strides = true;
  op->st = fa::Strides{sb, s.head, s.row};
  return FA_OK;
}

// A contiguous float32 statistics array of `n` values.
Operand stat_operand(const void* data, long long n) {
  Operand op;
  op.base = reinterpret_cast<uintptr_t>(data);
  op.ndims = 1;
  op.dims[0] = Dim{1, n};
  op.extent = n;
  op.esize = 4;
  return op;
}

// Dims with more than one index, by increasing stride.
int sorted_dims(const Operand& a, Dim* out) {
  int n = 0;
  for (int i = 0; i < a.ndims; ++i)
    if (a.dims[i].count > 1) out[n++] = a.dims[i];
  std::sort(out, out + n, [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
  return n;
}

// Every index maps to its own element: each stride exceeds the largest offset the smaller
// dimensions reach (a sufficient condition; it holds for every dense or sliced layout).
bool injective(const Operand& a) {
  Dim d[4];
  const int n = sorted_dims(a, d);
  long long reach = 0;
  for (int i = 0; i < n; ++i) {
    if (d[i].stride <= reach) return false;
    reach += (d[i].count - 1) * d[i].stride;
  }
  return true;
}

// Is delta (elements) a difference of two offsets of the nested map d[0..n) (increasing
// strides, each above the reach of the ones below)? At each level from the top, delta =
// a*stride + e with |e| <= reach below, so at most two values of a need a look.
bool representable(long long delta, const Dim* d, int n) {
  if (n == 0) return delta == 0;
  long long reach = 0;
  for (int i = 0; i < n - 1; ++i) reach += (d[i].count - 1) * d[i].stride;
  const Dim& top = d[n - 1];
  const long long lo = delta - reach, hi = delta + reach;
  // a in [ceil(lo / stride), floor(hi / stride)] and |a| < count
  auto fdiv = [](long long x, long long y) { return x >= 0 ? x / y : -((-x + y - 1) / y); };
  long long a0 = -fdiv(-lo, top.stride), a1 = fdiv(hi, top.stride);
  a0 = std::max(a0, -(top.count - 1));
  a1 = std::min(a1, top.count - 1);
  for (long long a = a0; a <= a1; ++a)
    if (representable(delta - a * top.stride, d, n - 1)) return true;
  return false;
}

// The two operands share no element (exactly when both are 16-bit with equal strides,
// by address ranges otherwise).
bool disjoint(const Operand& a, const Operand& b) {
  if (a.extent == 0 || b.extent == 0) return true;
  const uintptr_t alo = a.base, ahi = a.base + (uintptr_t)a.extent * a.esize;
  const uintptr_t blo = b.base, bhi = b.base + (uintptr_t)b.extent * b.esize;
  if (ahi <= blo || bhi <= alo) return true;
  if (!(a.has_strides && b.has_strides && a.esize == b.esize && a.ndims == b.ndims)) return false;
  for (int i = 0; i < a.ndims; ++i)
    if (a.dims[i].stride != b.dims[i].stride || a.dims[i].count != b.dims[i].count) return false;
  if (!injective(a)) return false;
  const long long bytes = (long long)(b.base - a.base);  // wraps to the signed difference
  if (bytes % a.esize != 0) return false;
  Dim d[4];
  const int n = sorted_dims(a, d);
  return !representable(bytes / a.esize, d, n);
}

// Outputs injective, disjoint from every input and from each other.
int check_overlaps(const Operand* ins, int nin, const Operand* outs, int nout) {
  for (int i = 0; i < nout; ++i) {
    if (outs[i].has_strides && !injective(outs[i])) return FA_ERR_INVALID_ARG;
    for (int j = 0; j < nin; ++j)
      if (!disjoint(outs[i], ins[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < nout; ++j)
      if (!disjoint(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

fa::Geom geom_of(const fa_problem& p) {
  fa::Geom g;
  g.B = p.B;
  g.H = p.H;
  g.N = p.N;
  g.cu = p.cu_seqlens;
  g.T = p.cu_seqlens ? p.total : 0;
  g.dh = p.d;
  g.Nk = nk_of(p);
  g.cuk = p.cu_seqlens ? cuk_of(p) : nullptr;
  g.Tk = p.cu_seqlens ? totalk_of(p) : 0;
  return g;
}

long long stat_count(const fa_problem& p) {
  return p.cu_seqlens ? (long long)p.H * p.total : (long long)p.B * p.H * p.N;
}

fa_strides contiguous(int H, int N, int d) {
  return fa_strides{(long long)H * N * d, (long long)N * d, (long long)d};
}

fa_problem fixed_problem(int B, int H, int N, int d, int causal, float scale, int dtype) {
  fa_problem p;
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.cu_seqlens = nullptr;
  p.total = 0;
  p.causal = causal;
  p.scale = scale;
  p.dtype = dtype;
  p.N_k = 0;
  p.cu_seqlens_k = nullptr;
  p.total_k = 0;
  return p;
}

// Most key ranges one Q tile may be cut into.
constexpr int kMaxSplits = 256;

// Width of the kernel that runs head dim d.
int kernel_d(int d) { return d <= 64 ? 64 : d <= 128 ? 128 : 256; }

// Bytes of split-KV workspace: per split and row, the kernel width's fp32 accumulators, a max
// and a sum.
long long splitkv_bytes(long long rows, int d, int splits) {
  return (long long)splits * rows * (kernel_d(d) + 2) * 4;
}

// Packed batches with no rows: the forward has no query; the backward also needs no key (a
// key no query sees still gets dK = dV = 0 written).
bool nothing_to_do_fwd(const fa_problem& p) { return p.cu_seqlens != nullptr && p.total == 0; }
bool nothing_to_do_bwd(const fa_problem& p) { return p.cu_seqlens != nullptr && p.total == 0 && totalk_of(p) == 0; }

int forward_impl(const fa_problem* pp, const void* q, const fa_strides& sq, const void* k, const fa_strides& sk,
                 const void* v, const fa_strides& sv, void* o, const fa_strides& so, float* lse, int splits,
                 float* part, size_t part_bytes, void* stream, bool pingpong = false) {
  if (!pp) return FA_ERR_INVALID_ARG;
  const fa_problem& p = *pp;
  int st = check_shape(p);
  if (st != FA_OK) return st;
  Operand ins[3], outs[3];
  if ((st = make_operand(p, q, sq, qrows(p), &ins[0])) != FA_OK) return st;
  if ((st = make_operand(p, k, sk, krows(p), &ins[1])) != FA_OK) return st;
  if ((st = make_operand(p, v, sv, krows(p), &ins[2])) != FA_OK) return st;
  if ((st = make_operand(p, o, so, qrows(p), &outs[0])) != FA_OK) return st;
  int nout = 1;
  const long long rows = stat_count(p);
  if (lse) {
    if (!aligned16(lse)) return FA_ERR_INVALID_ARG;
    outs[nout++] = stat_operand(lse, rows);
  }
  if (splits > 0) {
    if (!part || !aligned16(part)) return FA_ERR_INVALID_ARG;
    const long long need = splitkv_bytes(rows, p.d, splits);
    if ((unsigned long long)need > (unsigned long long)part_bytes) return FA_ERR_INVALID_ARG;
    outs[nout++] = stat_operand(part, need / 4);
    // grid = (N / 128 Q tiles) * splits * B*H workgroups in one 32-bit grid dimension
    if (((long long)p.N + 127) / 128 * splits * ((long long)p.B * p.H) > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  }
  if ((st = check_overlaps(ins, 3, outs, nout)) != FA_OK) return st;
  if (nothing_to_do_fwd(p)) return FA_OK;
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.sq = ins[0].st;
  a.sk = ins[1].st;
  a.sv = ins[2].st;
  a.so = outs[0].st;
  a.g = geom_of(p);
  a.d = p.d;
  a.causal = p.causal != 0;
  a.bf16 = p.dtype == FA_BF16;
  a.c_log2 = (float)((double)p.scale * kLog2eD);
  a.stream = stream;
  a.splits = splits;
  a.part = part;
  a.pingpong = pingpong;
  return fa::launch_forward(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Backward validation. Null pointers are operands a stage does not use (their strides are
// ignored); `delta` is an output of the stages that compute D from O (need_o: the preprocess
// stage, dQ with D, the whole backward) and an input otherwise.
int check_bwd(const fa_problem* pp, const void* q, const fa_strides& sq, const void* k, const fa_strides& sk,
              const void* v, const fa_strides& sv, const void* o, const fa_strides& so, const void* dO,
              const fa_strides& sdo, const float* lse, const void* dq, const fa_strides& sdq, const void* dk,
              const fa_strides& sdk, const void* dv, const fa_strides& sdv, const float* delta, bool need_qkv,
              bool need_o, bool need_dq, bool need_dkv, fa::BwdArgs* a) {
  if (!pp) return FA_ERR_INVALID_ARG;
  const fa_problem& p = *pp;
  if (!dO || !delta) return FA_ERR_INVALID_ARG;
  if (need_qkv && (!q || !k || !v || !lse)) return FA_ERR_INVALID_ARG;
  if (need_o && !o) return FA_ERR_INVALID_ARG;
  if (need_dq && !dq) return FA_ERR_INVALID_ARG;
  if (need_dkv && (!dk || !dv)) return FA_ERR_INVALID_ARG;
  if ((lse && !aligned16(lse)) || !aligned16(delta)) return FA_ERR_INVALID_ARG;
  int st = check_shape(p);
  if (st != FA_OK) return st;
  const long long rows = stat_count(p);
  Operand ins[7], outs[4];
  int nin = 0, nout = 0;
  Operand op;
  struct T16 {
    const void* data;
    const fa_strides* s;
    fa::Strides* dst;
    bool out, key_side;
  } t16[] = {{q, &sq, &a->sq, false, false},   {k, &sk, &a->sk, false, true},   {v, &sv, &a->sv, false, true},
             {o, &so, &a->so, false, false},   {dO, &sdo, &a->sdo, false, false}, {dq, &sdq, &a->sdq, true, false},
             {dk, &sdk, &a->sdk, true, true}, {dv, &sdv, &a->sdv, true, true}};
  for (const T16& t : t16) {
    *t.dst = fa::Strides{0, 0, 0};
    if (!t.data) continue;
    if ((st = make_operand(p, t.data, *t.s, t.key_side ? krows(p) : qrows(p), &op)) != FA_OK) return st;
    *t.dst = op.st;
    if (t.out)
      outs[nout++] = op;
    else
      ins[nin++] = op;
  }
  if (lse) ins[nin++] = stat_operand(lse, rows);
  if (need_o)
    outs[nout++] = stat_operand(delta, rows);
  else
    ins[nin++] = stat_operand(delta, rows);
  if ((st = check_overlaps(ins, nin, outs, nout)) != FA_OK) return st;
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
  a->g = geom_of(p);
  a->d = p.d;
  a->causal = p.causal != 0;
  a->bf16 = p.dtype == FA_BF16;
  a->scale = p.scale;
  a->c_log2 = (float)((double)p.scale * kLog2eD);
  return FA_OK;
}


}  // namespace

namespace fa {

bool pair_causal_tiles(long long paired_grid) {
  static std::atomic<int> cus[64];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus[dev].store(n, std::memory_order_relaxed);
  }
  return n <= 0 || paired_grid >= 2LL * n;
}

}  // namespace fa

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

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, int dtype, void* stream) {
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  return forward_impl(&p, q, c, k, c, v, c, o, c, lse, 0, nullptr, 0, stream);
}

int fa_forward_pingpong(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                        int d, int causal, float scale, int dtype, void* stream) {
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  return forward_impl(&p, q, c, k, c, v, c, o, c, lse, 0, nullptr, 0, stream, true);
}

int fa_forward_ex(const fa_problem* p, const void* q, fa_strides sq, const void* k, fa_strides sk, const void* v,
                  fa_strides sv, void* o, fa_strides so, float* lse, void* stream) {
  return forward_impl(p, q, sq, k, sk, v, sv, o, so, lse, 0, nullptr, 0, stream);
}

int fa_forward_splitkv_ex(const fa_problem* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
                          const void* v, fa_strides sv, void* o, fa_strides so, float* lse, int num_splits,
                          float* workspace, size_t workspace_bytes, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  return forward_impl(p, q, sq, k, sk, v, sv, o, so, lse, num_splits, workspace, workspace_bytes, stream);
}

size_t fa_forward_splitkv_ex_workspace_bytes(const fa_problem* p, int num_splits) {
  if (!p || num_splits < 1 || num_splits > kMaxSplits) return 0;
  if (check_shape(*p) != FA_OK) return 0;
  return (size_t)splitkv_bytes(stat_count(*p), p->d, num_splits);
}

size_t fa_forward_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  if (num_splits < 1 || num_splits > kMaxSplits) return 0;
  const fa_problem p = fixed_problem(B, H, N, d, 0, 1.0f, FA_BF16);
  if (check_shape(p) != FA_OK) return 0;
  return (size_t)splitkv_bytes(stat_count(p), d, num_splits);
}

int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       int d, int causal, float scale, int dtype, int num_splits, float* workspace,
                       size_t workspace_bytes, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  return forward_impl(&p, q, c, k, c, v, c, o, c, lse, num_splits, workspace, workspace_bytes, stream);
}

int fa_backward_ex(const fa_problem* p, const void* q, fa_strides sq, const void* k, fa_strides sk, const void* v,
                   fa_strides sv, const void* o, fa_strides so, const void* dO, fa_strides sdo, const float* lse,
                   void* dq, fa_strides sdq, void* dk, fa_strides sdk, void* dv, fa_strides sdv, float* delta,
                   void* stream) {
  fa::BwdArgs a;
  // delta is written by the first stage and read by the other two: validate it as an output.
  int st = check_bwd(p, q, sq, k, sk, v, sv, o, so, dO, sdo, lse, dq, sdq, dk, sdk, dv, sdv, delta, true, true,
                     true, true, &a);
  if (st != FA_OK) return st;
  if (nothing_to_do_bwd(*p)) return FA_OK;
  a.stream = stream;
  // dQ first: each of its workgroups also computes D for its own query rows and writes delta,
  // which the dK/dV stage then reads (the preprocess stage's work, without its extra pass
  // over dO)
  a.dq_delta = true;
  if (fa::launch_bwd_dq(a) != hipSuccess) return FA_ERR_HIP;
  a.dq_delta = false;
  if (fa::launch_bwd_dkv(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d, int causal, float scale,
                int dtype, void* stream) {
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  return fa_backward_ex(&p, q, c, k, c, v, c, o, c, dO, c, lse, dq, c, dk, c, dv, c, delta, stream);
}

int fa_backward_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d, int dtype,
                           void* stream) {
  fa::BwdArgs a;
  // the preprocess stage ignores causal and scale; validate them at neutral values
  const fa_problem p = fixed_problem(B, H, N, d, 0, 1.0f, dtype);
  const fa_strides c = contiguous(H, N, d);
  int st = check_bwd(&p, nullptr, c, nullptr, c, nullptr, c, o, c, dO, c, nullptr, nullptr, c, nullptr, c, nullptr,
                     c, delta, false, true, false, false, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  return fa::launch_bwd_preprocess(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dkv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                    const float* delta, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                    int dtype, void* stream) {
  fa::BwdArgs a;
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  int st = check_bwd(&p, q, c, k, c, v, c, nullptr, c, dO, c, lse, nullptr, c, dk, c, dv, c, delta, true, false,
                     false, true, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  return fa::launch_bwd_dkv(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                   const float* delta, void* dq, int B, int H, int N, int d, int causal, float scale, int dtype,
                   void* stream) {
  fa::BwdArgs a;
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  int st = check_bwd(&p, q, c, k, c, v, c, nullptr, c, dO, c, lse, dq, c, nullptr, c, nullptr, c, delta, true,
                     false, true, false, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dq_delta(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, float* delta, int B, int H, int N, int d, int causal,
                         float scale, int dtype, void* stream) {
  fa::BwdArgs a;
  const fa_problem p = fixed_problem(B, H, N, d, causal, scale, dtype);
  const fa_strides c = contiguous(H, N, d);
  // delta is an output here
  int st = check_bwd(&p, q, c, k, c, v, c, o, c, dO, c, lse, dq, c, nullptr, c, nullptr, c, delta, true, true, true,
                     false, &a);
  if (st != FA_OK) return st;
  a.stream = stream;
  a.dq_delta = true;
  return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
