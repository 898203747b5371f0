// Exact tiled attention backward for gfx950: three kernels, no atomics.
//
// "Triton 05: Flash Attention", sections "Backward 구현", "LSE로 P 재계산", "Softmax Gradient"
// and "3단계 커널 구조": P is rebuilt from the saved LSE (P_ij = exp(S_ij - LSE_i)), the
// softmax gradient is dS = P * (dP - D) with D_i = rowsum(dO_i * O_i) computed once, and the
// work is split so every output tile has exactly one writer:
//   [1] preprocess : D (here `delta`) from O and dO                      -- HBM-bound
//   [2] dK/dV      : one workgroup per K/V tile, loop over Q tiles (fa_bwd_dkv.hip)
//                    dV += P^T dO,  dP = dO V^T,  dS = P*(dP - D),  dK += scale * dS^T Q
//   [3] dQ         : one workgroup per Q tile (pinned in VGPRs), loop over K/V tiles
//                    dP = dO V^T,  dS = P*(dP - D),  dQ += scale * dS K
// All products run on the matrix cores with fp32 accumulation; P and dS are rounded to the
// input type (nearest even) as matrix-core operands. Operands whose contraction index runs
// down the rows of a staged tile (Q^T, dO^T, K^T) are read with the transposing LDS load.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

#include <type_traits>

namespace fa {

// ------------------------------------------------------------------------------------------
// [1] D_i = sum_c dO_ic * O_ic, fp32 accumulation, from the stored (rounded) O.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const uint16_t* __restrict__ O,
                                                             const uint16_t* __restrict__ dO,
                                                             float* __restrict__ delta, long long rows) {
  constexpr int TPR = D / 8;       // threads per row (16 B each)
  constexpr int RPB = 256 / TPR;   // rows per block per pass
  const int sub = threadIdx.x % TPR;
  long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const long long step = (long long)gridDim.x * RPB;
  for (; row < rows; row += step) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(O + row * D + sub * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + row * D + sub * 8);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = __builtin_fmaf(T::to_f32((uint16_t)(o[w] & 0xffff)), T::to_f32((uint16_t)(g[w] & 0xffff)), s);
      s = __builtin_fmaf(T::to_f32((uint16_t)(o[w] >> 16)), T::to_f32((uint16_t)(g[w] >> 16)), s);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (sub == 0) delta[row] = s;
  }
}

// ------------------------------------------------------------------------------------------
// [3] dQ. Workgroup = NW waves, each owning QB*32 query rows (Q, dO, LSE, D pinned); K/V
// tiles of BN keys are copied global -> LDS (swizzled) by the asynchronous loads into a
// double-buffered ring.
template <typename T, int D, int BN, int NW, int QB, int NBUF, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dQ, int BH, int N, int n_qtiles, float scale, float c_log2) {
  constexpr int BM = NW * QB * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = BN / 32;

  // K is read by rows (S^T) and transposed (dQ), V by rows: swizzled layout for both.
  // One array per ring slot: with every slot index a compile-time constant the compiler can
  // tell a copy into one slot from reads of another and does not wait for the copy first.
  static_assert(NBUF == 2, "ring of two slots");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps copy setup scalar
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // A head's Q tiles run together on one XCD (shared K/V reads in its L2), heaviest
  // causal tile first.
  const int lid = xcd_local_index(blockIdx.x, BH * n_qtiles);
  const int bh = __builtin_amdgcn_readfirstlane(lid / n_qtiles);  // wave-uniform (keeps pointers scalar)
  const int qt = __builtin_amdgcn_readfirstlane(CAUSAL ? (n_qtiles - 1 - lid % n_qtiles) : (lid % n_qtiles));
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QB * 32;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  auto stage = [&](int t, uint16_t* kdst, uint16_t* vdst) {
    stage_rows_swz_buf<D, BN, NW>(kdst, Kh, t * BN, N, wave);
    stage_rows_swz_buf<D, BN, NW>(vdst, Vh, t * BN, N, wave);
  };
  stage(0, lds_k0, lds_v0);

  Frag qf[QB][KS], dof[QB][KS];
  float lse2[QB], dl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + qb * 32 + l32;
    const bool ok = qrow < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks].v = gload16(Q + head + (size_t)qrow * D + ks * 16 + h * 8, ok);
      dof[qb][ks].v = gload16(dO + head + (size_t)qrow * D + ks * 16 + h * 8, ok);
    }
    lse2[qb] = ok ? LSE[(size_t)bh * N + qrow] * kLog2e : 0.f;
    dl[qb] = ok ? Delta[(size_t)bh * N + qrow] : 0.f;
  }

  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qb][db][i] = 0.f;

  // Per-lane fragment base offsets (every fragment address is one XOR / add away).
  const int rows0 = swz_rows_base<D>(0);
  const int cols0 = swz_cols_base<D>();

  wait_async();
  __syncthreads();

  // One K/V tile per call; `ks_base`/`vs_base` hold tile t, the other slot receives tile
  // t+1 (clamped: the prefetch is unconditional).
  auto tile_step = [&](int t, const uint16_t* ks_base, const uint16_t* vs_base, uint16_t* knext,
                       uint16_t* vnext) {
    stage(min(t + 1, ntiles - 1), knext, vnext);
    const int kbase = t * BN;
    // Every wave runs every K/V tile of the workgroup's range (fully masked tiles add 0;
    // that includes the padding step when the tile count is odd).
    const bool need_mask = (kbase + BN > N) || (CAUSAL && (kbase + BN - 1 > qw0));
    f32x16 s[QB][KB], dp[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[qb][kb][i] = 0.f;
          dp[qb][kb][i] = 0.f;
        }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Frag ak = swz_rows_frag<D>(ks_base, rows0 + kb * 32 * D, ks);
        const Frag av = swz_rows_frag<D>(vs_base, rows0 + kb * 32 * D, ks);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[qb][kb] = T::mfma(ak, qf[qb][ks], s[qb][kb]);
          dp[qb][kb] = T::mfma(av, dof[qb][ks], dp[qb][kb]);
        }
      }
    Frag dsf[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + qb * 32 + l32;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = __builtin_fmaf(s[qb][kb][i], c_log2, -lse2[qb]);
          // hidden entries get 2^-inf = 0 (a select on the exponent input, no branch)
          const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          // (bitwise, not short-circuit, operators: keeps this a select instead of branches)
          const bool hidden = need_mask & ((key >= N) | (CAUSAL & (key > qrow)));
          x = hidden ? -INFINITY : x;
          const float p = __builtin_amdgcn_exp2f(x);
          dp[qb][kb][i] = p * (dp[qb][kb][i] - dl[qb]);
        }
        dsf[qb][kb][0] = pack_group<T>(dp[qb][kb], 0);
        dsf[qb][kb][1] = pack_group<T>(dp[qb][kb], 1);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const Frag a = swz_cols_frag<D>(ks_base, cols0, kb * 32 + tt * 16, db * 32);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = T::mfma(a, dsf[qb][kb][tt], acc[qb][db]);
        }
    // Tile t+1 must have landed: allow the NBUF-2 younger tiles to stay in flight.
    // Tile t+1 must have landed before anyone reads it.
    wait_async();
    ring_barrier();
  };
  // Two steps per trip with the slots fixed at compile time; an odd tile count gets one
  // fully masked padding step (its keys are past the causal range or past N).
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(t, lds_k0, lds_v0, lds_k1, lds_v1);
    tile_step(t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  }
  // No copy may still be landing in LDS when the workgroup retires.
  wait_async();

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + qb * 32 + l32;
    if (qrow < N) {
      uint16_t* row = dQ + head + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = T::pack2(acc[qb][db][4 * g + 0] * scale, acc[qb][db][4 * g + 1] * scale);
          w[1] = T::pack2(acc[qb][db][4 * g + 2] * scale, acc[qb][db][4 * g + 3] * scale);
          *reinterpret_cast<u32x2*>(row + db * 32 + 8 * g + 4 * h) = w;
        }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Launchers.

template <typename T, int D>
static hipError_t launch_pre_t(const BwdArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const long long rows = (long long)a.BH * a.N;
  long long blocks = (rows + RPB - 1) / RPB;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((bwd_preprocess_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)a.stream,
                     (const uint16_t*)a.o, (const uint16_t*)a.dO, a.delta, rows);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a) {
  constexpr int NW = 4, QB = 1, BN = 32, NBUF = 2;
  constexpr int BM = NW * QB * 32;
  const int n_qtiles = (a.N + BM - 1) / BM;
  const long long grid = (long long)n_qtiles * a.BH;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, BN, NW, QB, NBUF, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dO, a.lse, a.delta, (uint16_t*)a.dq, a.BH, a.N, n_qtiles, a.scale,
                     a.c_log2);
  return hipGetLastError();
}

template <typename T>
static hipError_t pre_dt(const BwdArgs& a) {
  return a.d == 64 ? launch_pre_t<T, 64>(a) : launch_pre_t<T, 128>(a);
}
template <typename T>
static hipError_t dq_dt(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_dq_t<T, 64, true>(a) : launch_dq_t<T, 64, false>(a);
  return a.causal ? launch_dq_t<T, 128, true>(a) : launch_dq_t<T, 128, false>(a);
}

hipError_t launch_bwd_preprocess(const BwdArgs& a) { return a.bf16 ? pre_dt<BF16>(a) : pre_dt<FP16>(a); }
hipError_t launch_bwd_dq(const BwdArgs& a) { return a.bf16 ? dq_dt<BF16>(a) : dq_dt<FP16>(a); }

}  // namespace fa
