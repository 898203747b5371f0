// Exact tiled attention backward, stage [2]: dK and dV ("Triton 05: Flash Attention",
// sections "3단계 커널 구조" and "dKV 커널 수식": K_j and V_j stay on chip while every Q tile i
// streams past; each workgroup owns its dK_j, dV_j, so no atomics are needed).
//
// Per 32-query step and wave (32 keys): S = Q K^T and dP = dO V^T on the matrix cores
// (A = Q / dO rows from LDS, B = the wave's pinned K / V), P = 2^(c*S - LSE*log2 e) with the
// causal / tail mask folded into the exponent input, dS = P * (dP - D), then
// dV^T += dO^T P and dK^T += Q^T dS (A = transposing LDS reads, B = P / dS rounded to the
// input type). dK is scaled once at the end.
//
// Register plan (d = 128: one wave per SIMD): dK^T and dV^T accumulators (128), pinned K and
// V fragments (64), S, dP and operands in VGPRs. The step body is a single path -- the
// causal / tail mask is a select on the exponent input, evaluated every step -- because a
// masked and an unmasked copy of the body made the allocator copy the accumulators at the
// join on every iteration.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

#include <type_traits>

namespace fa {

// ------------------------------------------------------------------------------------------
// [2] dK, dV. Workgroup = NW waves, each owning 32 keys (K pinned in VGPRs, dK/dV
// accumulated in VGPRs); the workgroup's V tile sits in LDS for the whole kernel; Q/dO tiles
// of 32 rows and their LSE and D values stream through a double-buffered LDS ring, copied
// straight from global memory (no staging registers). Two workgroups fit a CU, so two waves
// share each SIMD and hide each other's latencies.
template <typename T, int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, float scale, float c_log2) {
  constexpr int BK = NW * 32;
  constexpr int BQ = 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;

  // The workgroup's V tile stays in LDS; Q/dO tiles stream. All tiles are swizzled (row and
  // transposed reads are both conflict-free).
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_q[2][BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_do[2][BQ * D];
  __shared__ __attribute__((aligned(256))) float lds_stat[2][64];  // [0,32): LSE, [32,64): D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // A head's K tiles run together on one XCD (shared Q/dO reads in its L2); causal: low
  // key tiles see the most queries and go first.
  const int n_ktiles = (N + BK - 1) / BK;
  const int lid = xcd_local_index(blockIdx.x, BH * n_ktiles);
  const int bh = lid / n_ktiles;
  const int kt = lid % n_ktiles;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* dOh = dO + head;
  const float* lse_h = LSE + (size_t)bh * N;
  const float* dl_h = Delta + (size_t)bh * N;

  const int it_begin = CAUSAL ? (k0 / BQ) : 0;
  const int it_end = (N + BQ - 1) / BQ;

  auto stage = [&](int it, int buf) {
    stage_rows_swz<D, BQ, NW>(lds_q[buf], Qh, it * BQ, N, wave);
    stage_rows_swz<D, BQ, NW>(lds_do[buf], dOh, it * BQ, N, wave);
    if (wave == NW - 1) stage_stats(lds_stat[buf], lse_h, dl_h, it * BQ, N);
  };

  stage_rows_swz<D, BK, NW>(lds_v, V + head, k0, N, wave);
  stage(it_begin, 0);

  // Pinned K fragments (B operand of S = Q K^T): lane holds K[key][16ks + 8h .. +7].
  Frag kf[KS];
  {
    const bool ok = key < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks].v = gload16(K + head + (size_t)key * D + ks * 16 + h * 8, ok);
  }
  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc_dk[db][i] = 0.f;
      acc_dv[db][i] = 0.f;
    }
  wait_async();
  __syncthreads();

  // Per-lane fragment base offsets (every fragment address is one XOR / add away).
  const int rows0 = swz_rows_base<D>(0);
  const int rows_v = swz_rows_base<D>(wave * 32);
  const int cols0 = swz_cols_base<D>();

  // One 32-query step; the mask handles the causal diagonal and the tails (q >= N, key >= N).
  auto step = [&](auto mask_tag, int it, int buf) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* qs = lds_q[buf];
    const uint16_t* dos = lds_do[buf];
    const int qbase = it * BQ;
    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = 0.f;
      dp[i] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = T::mfma(swz_rows_frag<D>(qs, rows0, ks), kf[ks], s);
      dp = T::mfma(swz_rows_frag<D>(dos, rows0, ks), swz_rows_frag<D>(lds_v, rows_v, ks), dp);
    }
    // rows of this lane: q_local = 8g + 4h + r for register i = 4g + r
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ql = 8 * g + 4 * h;
      const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&lds_stat[buf][ql]);
      const f32x4 dl4 = *reinterpret_cast<const f32x4*>(&lds_stat[buf][32 + ql]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        float x = __builtin_fmaf(s[i], c_log2, -lse4[r] * kLog2e);
        if (MASK) {
          // hidden entries get 2^-inf = 0 (a select on the exponent input, no branch)
          const int qrow = qbase + ql + r;
          const bool hidden = (qrow >= N) | (key >= N) | (CAUSAL & (key > qrow));
          x = hidden ? -INFINITY : x;
        }
        const float p = __builtin_amdgcn_exp2f(x);
        s[i] = p;
        dp[i] = p * (dp[i] - dl4[r]);
      }
    }
    const Frag pf0 = pack_group<T>(s, 0), pf1 = pack_group<T>(s, 1);
    const Frag df0 = pack_group<T>(dp, 0), df1 = pack_group<T>(dp, 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc_dv[db] = T::mfma(swz_cols_frag<D>(dos, cols0, 0, db * 32), pf0, acc_dv[db]);
      acc_dv[db] = T::mfma(swz_cols_frag<D>(dos, cols0, 16, db * 32), pf1, acc_dv[db]);
      acc_dk[db] = T::mfma(swz_cols_frag<D>(qs, cols0, 0, db * 32), df0, acc_dk[db]);
      acc_dk[db] = T::mfma(swz_cols_frag<D>(qs, cols0, 16, db * 32), df1, acc_dk[db]);
    }
  };

  for (int it = it_begin; it < it_end; ++it) {
    const int buf = (it - it_begin) & 1;
    // Prefetch unconditionally (the last step re-reads a valid tile into the idle buffer).
    stage(it + 1 < it_end ? it + 1 : it, buf ^ 1);
    step(std::integral_constant<bool, true>(), it, buf);
    wait_async();
    __syncthreads();
  }

  if (key < N) {
    uint16_t* dk_row = dK + head + (size_t)key * D;
    uint16_t* dv_row = dV + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk, wv;
        wk[0] = T::pack2(acc_dk[db][4 * g + 0] * scale, acc_dk[db][4 * g + 1] * scale);
        wk[1] = T::pack2(acc_dk[db][4 * g + 2] * scale, acc_dk[db][4 * g + 3] * scale);
        wv[0] = T::pack2(acc_dv[db][4 * g + 0], acc_dv[db][4 * g + 1]);
        wv[1] = T::pack2(acc_dv[db][4 * g + 2], acc_dv[db][4 * g + 3]);
        *reinterpret_cast<u32x2*>(dk_row + db * 32 + 8 * g + 4 * h) = wk;
        *reinterpret_cast<u32x2*>(dv_row + db * 32 + 8 * g + 4 * h) = wv;
      }
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_dkv_t(const BwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BK = NW * 32;
  const int n_ktiles = (a.N + BK - 1) / BK;
  const long long grid = (long long)n_ktiles * a.BH;
  hipLaunchKernelGGL((bwd_dkv_kernel<T, D, NW, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dO, a.lse, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.BH, a.N, a.scale,
                     a.c_log2);
  return hipGetLastError();
}

template <typename T>
static hipError_t dkv_dt(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_dkv_t<T, 64, true>(a) : launch_dkv_t<T, 64, false>(a);
  return a.causal ? launch_dkv_t<T, 128, true>(a) : launch_dkv_t<T, 128, false>(a);
}

hipError_t launch_bwd_dkv(const BwdArgs& a) { return a.bf16 ? dkv_dt<BF16>(a) : dkv_dt<FP16>(a); }

}  // namespace fa
