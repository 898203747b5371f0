/*
 * A C11 consumer of the library: include/fa.h compiles as C (not only as C++), libfa.so
 * links from C, and the host-side contracts hold when called from C: status strings, the
 * workspace-size formulas, and the argument checks that answer before any GPU work. Every
 * entry-point call below is built to fail validation (or is a pure size query), so the
 * made-up device addresses are never dereferenced and nothing is enqueued. Prints "ok" and
 * exits 0 on success; names the failed check and exits 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                            \
    }                                                                      \
  } while (0)

static void* addr(int i) { return (void*)(uintptr_t)((uintptr_t)(i + 1) << 28); }

int main(void) {
  void* q = addr(0);
  void* k = addr(1);
  void* v = addr(2);
  void* o = addr(3);
  float* lse = (float*)addr(4);
  void* dO = addr(5);
  void* dq = addr(6);
  void* dk = addr(7);
  void* dv = addr(8);
  float* delta = (float*)addr(9);

  /* status strings: static, never NULL, distinct for the four codes */
  CHECK(fa_status_string(FA_OK) != NULL && fa_status_string(99) != NULL);
  CHECK(strcmp(fa_status_string(FA_OK), fa_status_string(FA_ERR_INVALID_ARG)) != 0);
  CHECK(strcmp(fa_status_string(FA_ERR_UNSUPPORTED), fa_status_string(FA_ERR_HIP)) != 0);

  /* workspace sizes: num_splits * rows * (kernel width + 2) * 4, 0 when refused */
  CHECK(fa_forward_splitkv_workspace_bytes(2, 4, 100, 128, 3) == (size_t)3 * 2 * 4 * 100 * (128 + 2) * 4);
  CHECK(fa_forward_splitkv_workspace_bytes(1, 1, 10, 40, 2) == (size_t)2 * 10 * (64 + 2) * 4);
  CHECK(fa_forward_splitkv_workspace_bytes(1, 1, 10, 256, 1) == (size_t)10 * (256 + 2) * 4);
  CHECK(fa_forward_splitkv_workspace_bytes(1, 1, 10, 100, 2) == 0); /* head dim not a multiple of 8 */
  CHECK(fa_forward_splitkv_workspace_bytes(1, 1, 10, 64, 0) == 0);

  fa_problem p;
  memset(&p, 0, sizeof p);
  p.B = 2;
  p.H = 3;
  p.N = 1;
  p.d = 128;
  p.scale = 0.125f;
  p.dtype = FA_BF16;
  p.causal = 1;
  p.N_k = 4096; /* decode: one query row against 4096 keys */
  CHECK(fa_forward_splitkv_ex_workspace_bytes(&p, 8) == (size_t)8 * 2 * 3 * 1 * (128 + 2) * 4);
  CHECK(fa_forward_splitkv_ex_workspace_bytes(NULL, 8) == 0);

  /* argument checks (each call is refused before anything is enqueued) */
  CHECK(fa_forward(NULL, k, v, o, lse, 1, 1, 16, 64, 0, 0.125f, FA_FP16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward(q, k, v, o, lse, 1, 1, 16, 64, 0, 0.0f, FA_FP16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward(q, k, v, o, lse, 1, 1, 16, 64, 2, 0.125f, FA_FP16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward(q, k, v, o, lse, 1, 1, 16, 64, 0, 0.125f, 7, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward(q, k, v, q, lse, 1, 1, 16, 64, 0, 0.125f, FA_FP16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward_pingpong(NULL, k, v, o, lse, 1, 1, 16, 128, 0, 0.125f, FA_BF16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward_pingpong(q, k, v, q, lse, 1, 1, 16, 128, 1, 0.125f, FA_BF16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward_pingpong(q, k, v, o, lse, 1, 1, 16, 132, 0, 0.125f, FA_BF16, NULL) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward(q, k, v, o, lse, 1, 1, 16, 100, 0, 0.125f, FA_FP16, NULL) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward(q, k, v, o, lse, 1, 1, 16, 264, 0, 0.125f, FA_BF16, NULL) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward(q, k, v, o, dO, lse, dq, dk, dv, NULL, 1, 1, 16, 64, 1, 0.125f, FA_BF16, NULL) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_backward(q, k, v, o, dO, lse, dq, dq, dv, delta, 1, 1, 16, 64, 1, 0.125f, FA_BF16, NULL) ==
        FA_ERR_INVALID_ARG); /* two outputs on one buffer */
  CHECK(fa_backward_preprocess(o, dO, NULL, 1, 1, 16, 64, FA_BF16, NULL) == FA_ERR_INVALID_ARG);
  CHECK(fa_backward_dkv(q, k, v, dO, lse, delta, dk, NULL, 1, 1, 16, 64, 1, 0.125f, FA_BF16, NULL) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_backward_dq(q, k, v, dO, lse, delta, NULL, 1, 1, 16, 64, 1, 0.125f, FA_BF16, NULL) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_backward_dq_delta(q, k, v, NULL, dO, lse, dq, delta, 1, 1, 16, 64, 1, 0.125f, FA_BF16, NULL) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_backward_dq_delta(q, k, v, o, dO, lse, dq, delta, 1, 1, 16, 72 + 1, 1, 0.125f, FA_BF16, NULL) ==
        FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_splitkv(q, k, v, o, lse, 1, 1, 16, 64, 0, 0.125f, FA_FP16, 0, (float*)addr(10), 1 << 20,
                           NULL) == FA_ERR_INVALID_ARG); /* zero splits */

  fa_strides s = {4096LL * 3 * 128, 128, 3 * 128}; /* (B, N, H, d) storage */
  fa_strides sk = s;
  CHECK(fa_forward_ex(NULL, q, s, k, sk, v, sk, o, s, lse, NULL) == FA_ERR_INVALID_ARG);
  p.N_k = -1;
  CHECK(fa_forward_ex(&p, q, s, k, sk, v, sk, o, s, lse, NULL) == FA_ERR_INVALID_ARG);
  p.N_k = 4096;
  sk.row = 64; /* row stride below d */
  CHECK(fa_forward_ex(&p, q, s, k, sk, v, s, o, s, lse, NULL) == FA_ERR_INVALID_ARG);
  sk = s;
  CHECK(fa_forward_splitkv_ex(&p, q, s, k, sk, v, sk, o, s, lse, 8, (float*)addr(10), 16, NULL) ==
        FA_ERR_INVALID_ARG); /* workspace too small */
  p.cu_seqlens_k = (const int*)addr(11); /* key offsets without query offsets */
  CHECK(fa_backward_ex(&p, q, s, k, sk, v, sk, o, s, dO, s, lse, dq, s, dk, sk, dv, sk, delta, NULL) ==
        FA_ERR_INVALID_ARG);

  printf("ok\n");
  return 0;
}
