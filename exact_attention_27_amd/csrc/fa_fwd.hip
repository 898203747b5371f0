// Exact tiled attention forward for gfx950 (CDNA4).
//
// What it computes: O = softmax(scale * Q K^T, optional causal mask) V and the natural-log
// row LSE, never writing S or P anywhere ("Triton 05: Flash Attention", sections
// "Online Softmax", "코드 라인별 설명 (Forward)", "최종 정규화"; "GPU에서 Attention은 실제로
// 어떻게 실행되는가", sections 2-1..2-3 and 3-2).
//
// Work split (Q-outer, as in the FA2 walk-through, section 2-1): one workgroup per
// (batch*head, Q tile of BM rows); each of its NW waves owns QB*32 whole query rows
// ("split-Q", section 2-3), so row statistics never leave the wave. The K/V tiles of BN keys
// stream through a double-buffered LDS ring: the next tile's global loads are in flight while
// the current tile is consumed.
//
// Per K/V tile and wave:
//   S^T = K Q^T on the matrix cores (A = K rows from LDS, B = the wave's Q held in VGPRs),
//       so each lane owns one query column -> row max / row sum are in-lane plus one
//       cross-half exchange;
//   online softmax in base 2 (the exp -> exp2 trick, "Triton 05", section "exp → exp2 트릭"):
//       m' = max(m, c * max_j s_j), c = scale * log2(e); alpha = 2^(m - m');
//       p = 2^(c*s - m'); l = alpha*l + sum p; acc *= alpha;
//   O^T += V^T P^T on the matrix cores (A = V^T via transposing LDS reads, B = P converted
//       in registers, round to nearest even).
// Epilogue: divide once by l ("Triton 05", "최종 정규화"), store O and
// LSE = ln2 * (m + log2 l).
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Largest tolerated excess of a tile's max over the reference max, in log2 units: p <= 2^8.
constexpr float kTau = 8.0f;

template <typename T, int D, int BN, int NW, int QB, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int N, int n_qtiles, float c_log2) {
  constexpr int BM = NW * QB * 32;     // query rows per workgroup
  constexpr int KS = D / 16;           // k-steps over the head dim
  constexpr int DB = D / 32;           // 32-wide blocks of the head dim
  constexpr int KB = BN / 32;          // 32-key blocks per tile
  constexpr int SK = D + 8;            // LDS row stride of the K tile (elements)
  constexpr int SV = D + 32;           // LDS row stride of the V tile (elements)
  constexpr int NT = NW * 64;
  constexpr int CHUNKS = BN * D / 8;   // 16-byte chunks per K (or V) tile
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly over the workgroup");
  constexpr int CPT = CHUNKS / NT;
  constexpr int CPR = D / 8;           // chunks per row

  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BN * SK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][BN * SV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // A head's Q tiles run together on one XCD (shared K/V reads in its L2), heaviest
  // causal tile first.
  const int lid = xcd_local_index(blockIdx.x, BH * n_qtiles);
  const int bh = lid / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - lid % n_qtiles) : (lid % n_qtiles);
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QB * 32;  // first row of this wave

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qrow][16ks + 8h .. +7].
  Frag qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + qb * 32 + l32;
    const bool ok = qrow < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks].v = gload16(Qh + (size_t)qrow * D + ks * 16 + h * 8, ok);
  }

  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qb][db][i] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;  // per-lane partial sum over this lane's keys; halves merged at the end
  }

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  u32x4 pk[CPT], pv[CPT];
  auto gload_tile = [&](int t) {
    const int kbase = t * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, col = (c % CPR) * 8;
      const bool ok = kbase + row < N;
      pk[i] = gload16(Kh + (size_t)(kbase + row) * D + col, ok);
      pv[i] = gload16(Vh + (size_t)(kbase + row) * D + col, ok);
    }
  };
  auto lds_store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, col = (c % CPR) * 8;
      *reinterpret_cast<u32x4*>(&lds_k[buf][row * SK + col]) = pk[i];
      *reinterpret_cast<u32x4*>(&lds_v[buf][row * SV + col]) = pv[i];
    }
  };

  gload_tile(0);
  lds_store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // Prefetch unconditionally (the last iteration re-reads a valid tile into the idle
    // buffer): predicated loads would turn the staging registers into loop phis.
    gload_tile(t + 1 < ntiles ? t + 1 : t);
    const int kbase = t * BN;
    // Every wave runs every tile of the workgroup's range (a tile entirely above this
    // wave's rows is fully masked and adds p = 0), which keeps the loop body free of
    // branches around the accumulators.
    {
      const bool need_mask = (kbase + BN > N) || (CAUSAL && (kbase + BN - 1 > qw0));
      const uint16_t* ks_base = lds_k[buf];
      const uint16_t* vs_base = lds_v[buf];

      // ---- S^T = K Q^T
      f32x16 s[QB][KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[qb][kb][i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frag a = lds_frag_rows(ks_base, SK, kb * 32, ks * 16);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = T::mfma(a, qf[qb][ks], s[qb][kb]);
        }
      }

      // ---- mask (diagonal / tail tiles only)
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qrow = qw0 + qb * 32 + l32;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kbase + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
              const bool hidden = (key >= N) || (CAUSAL && key > qrow);
              if (hidden) s[qb][kb][i] = -INFINITY;
            }
        }
      }

      // ---- online softmax (base 2) with a lazily moved reference max.
      // The reference m_ref only moves when a tile's max exceeds it by more than kTau (log2
      // units); otherwise p = 2^(c*s - m_ref) <= 2^kTau is accumulated against the old
      // reference. O = acc / l and LSE = ln2 * (m_ref + log2 l) are exact for any reference
      // shared by acc and l, so this only skips rescales of the O accumulator (held in
      // AGPRs, where each rescale costs a read-modify-write of all of it). The branch is
      // wave-uniform: one lane that needs a move rescales the wave, with alpha = 1 for the
      // lanes whose reference stays.
      Frag p[QB][KB][2];
      bool moved = false;
      float alpha[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb][i]);
        mx = wave_xor32_max(mx) * c_log2;
        const bool move = mx > m_run[qb] + kTau;
        const float m_new = move ? mx : m_run[qb];
        moved |= move;
        alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);  // 1 if kept, 0 from -inf
        m_run[qb] = m_new;
        // A row that has seen no visible key keeps m = -inf; use 0 as the reference then.
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][i], c_log2, -m_ref));
            s[qb][kb][i] = e;
            rs += e;
          }
        l_run[qb] = l_run[qb] * alpha[qb] + rs;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          p[qb][kb][0] = pack_group<T>(s[qb][kb], 0);
          p[qb][kb][1] = pack_group<T>(s[qb][kb], 1);
        }
      }
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha[qb];
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            Frag a = lds_frag_cols(vs_base, SV, kb * 32 + tt * 16, db * 32);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = T::mfma(a, p[qb][kb][tt], acc[qb][db]);
          }
    }
    lds_store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: one division per row, store O and LSE
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + qb * 32 + l32;
    const float l_tot = wave_xor32_sum(l_run[qb]);
    const float inv = 1.0f / l_tot;
    if (qrow < N) {
      uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = T::pack2(acc[qb][db][4 * g + 0] * inv, acc[qb][db][4 * g + 1] * inv);
          w[1] = T::pack2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = w;
        }
      if (LSE != nullptr && h == 0) LSE[(size_t)bh * N + qrow] = (m_run[qb] + __log2f(l_tot)) * kLn2;
    }
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  constexpr int NW = 4, QB = 1, BN = 64;
  constexpr int BM = NW * QB * 32;
  const int n_qtiles = (a.N + BM - 1) / BM;
  const long long grid = (long long)n_qtiles * a.BH;
  hipLaunchKernelGGL((fwd_kernel<T, D, BN, NW, QB, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.BH, a.N, n_qtiles, a.c_log2);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fwd_dt(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_fwd_t<T, 64, true>(a) : launch_fwd_t<T, 64, false>(a);
  return a.causal ? launch_fwd_t<T, 128, true>(a) : launch_fwd_t<T, 128, false>(a);
}

hipError_t launch_forward(const FwdArgs& a) {
  return a.bf16 ? launch_fwd_dt<BF16>(a) : launch_fwd_dt<FP16>(a);
}

}  // namespace fa
