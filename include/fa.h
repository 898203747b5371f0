/*
 * fa.h -- C ABI of the exact IO-aware tiled attention library (libfa.so), gfx950.
 *
 * The library computes exact softmax attention, forward and backward, without
 * materialising the N x N score or probability matrices:
 *
 *   forward   O = softmax(scale * Q K^T  [causal mask]) V,  plus the row log-sum-exp
 *             LSE_i = m_i + ln(sum_j exp(S_ij - m_i)) (natural log), and nothing else.
 *             Defined on "Triton 05: Flash Attention" (wonbeomjang.kr), sections
 *             "Online Softmax", "코드 라인별 설명 (Forward)" and "LSE로 P 재계산";
 *             the result is the standard attention result, not an approximation
 *             ("FlashAttentionを1から", section "オンラインsoftmax").
 *   backward  dQ, dK, dV for an upstream gradient dO, recomputing P = exp(S - LSE)
 *             from the saved LSE and using D_i = rowsum(dO_i * O_i), in three stages
 *             (D; dK/dV with a pinned K/V tile; dQ with a pinned Q tile) so that every
 *             output tile has exactly one writer and no atomics are used ("Triton 05:
 *             Flash Attention", sections "Softmax Gradient" and "3단계 커널 구조");
 *             fa_backward runs the D stage inside the dQ kernel, in two launches.
 *
 * Conventions shared by every entry point:
 *
 *   Layout     Q, K, V, O, dO, dQ, dK, dV are contiguous row-major (B, H, N, d)
 *              tensors of the element type `dtype`; LSE and delta are contiguous
 *              (B, H, N) float32. fa_forward_ex / fa_backward_ex (end of this file)
 *              also take strided operands and variable-length batches.
 *   Types      dtype FA_FP16 (IEEE binary16) or FA_BF16 (bfloat16). Arithmetic is
 *              fp32 inside (fp32 accumulation on the matrix cores); every fp32 ->
 *              16-bit conversion rounds to nearest even. The forward's row sum of P is
 *              taken over fp32 P, except for fp16 at d <= 64, where it sums (in fp32) the
 *              P rounded to fp16 that the P V product uses: LSE then moves by at most
 *              2^-11 (about 4.9e-4) against the fp32 sum.
 *   Shapes     B, H, N >= 1; head dim d a multiple of 8 up to 256 (d <= 64 runs on the
 *              64-wide kernels, d <= 128 on the 128-wide ones, larger d on the 256-wide
 *              ones, with the columns past d zero on chip: exact, at the cost of the
 *              padded products). Any N is accepted (tails are masked). Other head dims
 *              (above 256, or not a multiple of 8) return FA_ERR_UNSUPPORTED -- never a
 *              slower or approximate fallback; the pages note that flash kernels cap the
 *              head dim ("FlashAttentionを1から", section "現場ではこう使う").
 *   Mask       causal = 0 (none) or 1: key j is visible to query i iff j <= i
 *              ("Triton 05", section "Causal Masking"; Nq = Nk so top-left and
 *              bottom-right alignment coincide).
 *   Scale      finite and > 0 (1/sqrt(d) for standard attention).
 *   Memory     all pointers are DEVICE pointers owned by the caller, 16-byte aligned.
 *              The library never allocates, frees or retains caller memory. Its global
 *              state is a per-device cache of the CU count, filled on first use with
 *              atomic stores, and, for fa_backward_noalloc only, a fixed device array per
 *              GPU with its cached address: calls are re-entrant (fa_backward_noalloc calls
 *              that overlap in time on one GPU excepted). Outputs must not overlap inputs or
 *              each other.
 *   Streams    `stream` is a hipStream_t (NULL = the default stream). All work is
 *              enqueued on it and the call returns without synchronising; buffers
 *              must stay alive until the stream reaches that point. Every pointer
 *              must be memory of the stream's device, and that device must be the
 *              calling thread's current one. The launch shape depends on the current
 *              device's CU count.
 *   Errors     arguments are validated on the host before anything is enqueued:
 *              FA_ERR_INVALID_ARG for null/misaligned/overlapping pointers,
 *              non-positive sizes, 64-bit size overflow, unknown dtype, a causal
 *              flag other than 0/1, or a non-finite / non-positive scale;
 *              FA_ERR_UNSUPPORTED for a valid request the library does not implement
 *              (head dim above 256 or not a multiple of 8); FA_ERR_HIP if one of this call's
 *              kernel launches fails (each launch's own status: an error left pending on the
 *              thread by an earlier, unrelated HIP call is not reported as this call's).
 *              Faults during execution surface at the caller's next synchronisation, as
 *              usual for HIP.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_FP16 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_HIP = 3
} fa_status;

/*
 * Forward pass.
 *   q, k, v  in : (B, H, N, d) dtype.
 *   o        out: (B, H, N, d) dtype, fully overwritten.
 *   lse      out: (B, H, N) float32, natural-log row log-sum-exp of the scaled,
 *                 masked scores; fully overwritten. May be NULL when no backward
 *                 pass will follow (inference); then it is not written.
 * One kernel launch. Returns an fa_status.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, int dtype,
               void* stream);

/*
 * fa_forward() with the two-group ping-pong schedule: the matrix product of one query
 * sub-tile overlaps the softmax of another ("FlashAttention·FA4·FP4", section "HBM을 아낀
 * 뒤에는 무엇이 기다리는가"; "Triton 05: Flash Attention", section "4. H100, B200에서의 추가
 * 기법"). For 64 < d <= 128 one workgroup of eight waves holds 256 query rows in two groups
 * of four, one group half a step behind the other, so each SIMD pairs one wave's
 * exponentials with the other's products. Other head dims run the schedule of fa_forward().
 * Arguments, outputs and errors are those of fa_forward(), and the outputs are bit-identical
 * to it (every row goes through the same operations in the same order). On MI355X it measured
 * slower than fa_forward() at the shapes tried; it is kept for comparison and for hardware
 * where the pairing pays.
 */
int fa_forward_pingpong(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        void* stream);

/*
 * Split-KV forward, for grids that would not fill the GPU (few heads, short sequences):
 * the keys of every 128-row Q tile are cut into `num_splits` contiguous ranges of 64-key
 * tiles, one workgroup each computes the softmax state (max m, sum l, unnormalised output)
 * of its range, and a second kernel merges the states -- the combination of partial
 * (m, l, O~) over disjoint key ranges described in "FlashAttentionを1から", section
 * "その後の版と、推論での事情". The result is the same exact attention as fa_forward
 * (same o and lse contract), up to fp32 rounding order.
 *   num_splits    1 .. 256; ranges beyond a tile's key count are empty and merge with
 *                 weight zero.
 *   workspace     device float32 scratch of at least
 *                 fa_forward_splitkv_workspace_bytes(B, H, N, d, num_splits) bytes,
 *                 16-byte aligned, not overlapping any other argument; contents on entry
 *                 are ignored and on return are unspecified.
 * Two kernel launches on `stream`. Returns an fa_status; a workspace that is NULL,
 * misaligned, too small or overlapping, or num_splits outside 1..256, is
 * FA_ERR_INVALID_ARG.
 */
int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale, int dtype,
                       int num_splits, float* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Workspace bytes fa_forward_splitkv needs: num_splits * B*H*N * (w + 2) * 4, where w = 64
 * for d <= 64, 128 for d <= 128 and 256 above (the width of the kernel that runs d). Returns 0 for
 * arguments fa_forward_splitkv would refuse (sizes, head dim, num_splits).
 */
size_t fa_forward_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits);

/*
 * Backward pass.
 *   q, k, v  in : the forward inputs.
 *   o, lse   in : the forward outputs for the same (scale, causal).
 *   dO       in : (B, H, N, d) dtype, gradient of the loss w.r.t. O.
 *   dq,dk,dv out: (B, H, N, d) dtype, fully overwritten (no zero-fill needed).
 *   delta    out: (B, H, N) float32 caller-provided workspace; on return (in stream
 *                 order) it holds D_i = sum_c dO_ic * O_ic, computed from the stored
 *                 O. Must not be NULL.
 * Two kernel launches on `stream`, in order: dQ, whose workgroups also compute D for their
 * own query rows and write delta (fa_backward_dq_delta), then dK/dV (fa_backward_dkv).
 * Returns an fa_status.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse, void* dq, void* dk, void* dv,
                float* delta, int B, int H, int N, int d, int causal, float scale,
                int dtype, void* stream);

/*
 * The backward stages, individually, for callers that interleave their own work or time each
 * kernel. Arguments have the same meaning, rules and errors as in fa_backward(). The pages
 * split the backward into three kernels ("Triton 05", "3단계 커널 구조"); fa_backward() runs
 * the first inside the third, as fa_backward_dq_delta then fa_backward_dkv on one stream.
 *   fa_backward_preprocess  delta_i = sum_c dO_ic * O_ic (stage 1). Reads o, dO; writes delta.
 *   fa_backward_dkv         dK, dV with one K/V tile pinned per workgroup, looping over Q
 *                           tiles (stage 2). Reads q, k, v, dO, lse, delta; writes dk, dv.
 *   fa_backward_dq          dQ with one Q tile pinned per workgroup, looping over K/V tiles
 *                           (stage 3). Reads q, k, v, dO, lse, delta; writes dq.
 *   fa_backward_dq_delta    stages 1 and 3 in one launch: each dQ workgroup computes D for its
 *                           own query rows from o and dO (the definition of stage 1, fp32),
 *                           writes it to delta and uses it. Reads q, k, v, o, dO, lse; writes
 *                           dq, delta. Its D (and so dq) may differ from the two-launch form by
 *                           fp32 summation order.
 */
int fa_backward_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d,
                           int dtype, void* stream);
int fa_backward_dkv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                    const float* delta, void* dk, void* dv, int B, int H, int N, int d, int causal,
                    float scale, int dtype, void* stream);
int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                   const float* delta, void* dq, int B, int H, int N, int d, int causal, float scale,
                   int dtype, void* stream);
int fa_backward_dq_delta(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, float* delta, int B, int H,
                         int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * Strided operands and variable-length batches.
 *
 * fa_strides: element strides of one operand. Element (b, h, r, c) of a (B, H, N, d)
 *   operand sits at data + b*batch + h*head + r*row + c: the d elements of a row are
 *   contiguous, the rest is the caller's choice. Examples: (B, H, N, d) storage is
 *   {H*N*d, N*d, d}; (B, N, H, d) storage is {N*H*d, d, H*d}; Q, K, V packed
 *   as (B, N, 3, H, d) share {3*N*H*d, d, 3*H*d} with data pointers H*d elements apart.
 *   Every stride is >= 0 and a multiple of 8 elements (16 bytes); row lies in [d, 2^23].
 *
 * fa_problem: the shape of one call.
 *   B, H, d, causal, scale, dtype  as for fa_forward().
 *   N_k   key rows per sequence when they differ from the query rows (0: N_k = N). The
 *         query-side operands (q, o, dO, dq; lse, delta) have N rows, the key-side ones
 *         (k, v, dk, dv) N_k. With the causal mask the queries are the last N of the
 *         N_k positions: query i sees key j iff j <= i + (N_k - N) (bottom-right; with
 *         N = N_k this is j <= i). A query that sees no key (N > N_k) gets O = 0,
 *         LSE = -inf and dQ = 0; a key no query sees gets dK = dV = 0. Decode is N = 1:
 *         one new token against the whole cache ("FlashAttentionを1から", section
 *         "その後の版と、推論での事情"), best served by fa_forward_splitkv_ex.
 *   cu_seqlens == NULL  every sequence has N rows; lse and delta are (B, H, N) float32.
 *   cu_seqlens != NULL  variable lengths ("FlashAttentionを1から", section "現場ではこう使う":
 *       padding every sequence to the longest pays for the padding; cumulative sequence
 *       offsets avoid it). A DEVICE array of B+1 int32 with
 *       0 = cu[0] <= cu[1] <= ... <= cu[B] = total: sequence b is the packed rows
 *       [cu[b], cu[b+1]) of every operand (each operand holds `total` rows of H heads; the
 *       batch stride is ignored). N is an upper bound of every length (the grid is sized
 *       by it); lse and delta are (H, total) float32. Each sequence attends only to itself.
 *       Key-side rows follow cu_seqlens_k (B+1 offsets, total_k rows in all, lengths at
 *       most N_k) when it is not NULL, else cu_seqlens. The library never reads these
 *       arrays on the host: offsets outside [0, total] ([0, total_k]) are clamped and
 *       lengths above N (N_k) cut on the device, so no contents make a kernel read or
 *       write outside the operands, but a batch that breaks the rules above gets
 *       unspecified values. total may be 0 (then the forward enqueues nothing).
 *
 * Overlap rules: outputs (o, lse; dq, dk, dv, delta) must address every element once
 * (injective strides) and share no element with any input or with each other. Inputs may
 * overlap each other. Two operands with equal strides are tested element-exactly (so the
 * three slices of one packed (B, N, 3, H, d) gradient are accepted as separate outputs);
 * otherwise their address ranges must not intersect.
 */
typedef struct {
  long long batch, head, row;
} fa_strides;

typedef struct {
  int B, H, N, d;
  const int* cu_seqlens;
  int total;
  int causal;
  float scale;
  int dtype;
  int N_k;                 /* 0: equal to N */
  const int* cu_seqlens_k; /* NULL: equal to cu_seqlens */
  int total_k;             /* with cu_seqlens_k: packed key rows in all */
} fa_problem;

/* fa_forward() on strided operands / variable-length batches (rules above). */
int fa_forward_ex(const fa_problem* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
                  const void* v, fa_strides sv, void* o, fa_strides so, float* lse, void* stream);

/* fa_backward() on strided operands / variable-length batches (rules above): the same two
 * kernels in the same order on `stream`. */
int fa_backward_ex(const fa_problem* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
                   const void* v, fa_strides sv, const void* o, fa_strides so, const void* dO,
                   fa_strides sdo, const float* lse, void* dq, fa_strides sdq, void* dk,
                   fa_strides sdk, void* dv, fa_strides sdv, float* delta, void* stream);

/*
 * The split-KV forward (fa_forward_splitkv) on a problem of the form above: every Q tile's
 * key tiles are cut into num_splits ranges. Decode shapes (N = 1, long N_k) fill the GPU
 * only this way. workspace: device float32 of at least
 * fa_forward_splitkv_ex_workspace_bytes(p, num_splits) bytes (num_splits * query rows *
 * (w + 2) * 4, w = the kernel width of d), same rules as for fa_forward_splitkv.
 * Choosing num_splits: about 256 workgroups in all did best in measurements on MI355X,
 * i.e. num_splits ~ 256 / (B * H * ceil(N / 128)), at least 1. More ranges add fixed cost
 * per range; fewer leave CUs idle.
 */
int fa_forward_splitkv_ex(const fa_problem* p, const void* q, fa_strides sq, const void* k, fa_strides sk,
                          const void* v, fa_strides sv, void* o, fa_strides so, float* lse, int num_splits,
                          float* workspace, size_t workspace_bytes, void* stream);
size_t fa_forward_splitkv_ex_workspace_bytes(const fa_problem* p, int num_splits);

/*
 * fa_backward() for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid allocation. The arguments
 * are those of fa_backward() without `delta`: the per-row vector D_i = rowsum(dO_i * O_i) that
 * the three kernels pass between them lives in a float32 array the library holds in device
 * memory, one per GPU for the life of the process, of fa_backward_noalloc_max_rows() rows
 * (2^22: 16 MiB). The call allocates nothing and makes no allocating library call; outputs and
 * errors are those of fa_backward() (dq, dk, dv bit-identical to it), plus
 * FA_ERR_UNSUPPORTED when B*H*N exceeds the array. The array's device address is looked up
 * once per device, on the first call with that device current (FA_ERR_HIP if the lookup
 * fails). Every call on one GPU shares its array: calls that overlap in time on one GPU (on
 * two streams, say) race on it and must be serialised by the caller. Nothing in the array has
 * to start at zero (each call's first kernel writes every row the other two read).
 */
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dO, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        void* stream);
size_t fa_backward_noalloc_max_rows(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
