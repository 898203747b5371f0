// Exact tiled attention backward for gfx950: three stages, no atomics.
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
// Stage [1] also runs inside [3]: given O, each dQ workgroup computes D for the query rows it
// owns (it holds their dO already) and writes it, so the full backward is [3] then [2], two
// launches, with no separate pass over O and dO.
// All products run on the matrix cores with fp32 accumulation; P and dS are rounded to the
// input type (nearest even) as matrix-core operands. Operands whose contraction index runs
// down the rows of a staged tile (Q^T, dO^T, K^T) are read with the transposing LDS load.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

#include <type_traits>

namespace fa {

// ------------------------------------------------------------------------------------------
// [1] D_i = sum_c dO_ic * O_ic, fp32 accumulation, from the stored (rounded) O. A block covers
// pre_rows_per_block<D>() consecutive rows of one statistics head (nrb blocks per head): each
// thread issues the loads of its PASSES rows (16 B of O and of dO each) before using any, so
// a CU keeps enough bytes in flight to run at the HBM rate rather than at its latency.
constexpr int kPrePasses = 4;
template <int D>
constexpr int pre_rows_per_block() { return kPrePasses * 256 / (D / 8); }

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const uint16_t* __restrict__ O,
                                                             const uint16_t* __restrict__ dO,
                                                             float* __restrict__ delta, Geom geo, Strides so,
                                                             Strides sdo, int nrb) {
  constexpr int TPR = D / 8;       // threads per row (16 B each)
  constexpr int RPP = 256 / TPR;   // rows per pass
  const int sub = threadIdx.x % TPR;
  const int hh = blockIdx.x / nrb;
  const int r0 = (blockIdx.x - hh * nrb) * pre_rows_per_block<D>() + threadIdx.x / TPR;
  const int rows = stat_rows(geo);
  // chunks past the operands' head dim, and rows past the head, count as zero
  const bool inside = sub * 8 < geo.dh;
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 o[kPrePasses], g[kPrePasses];
#pragma unroll
  for (int p = 0; p < kPrePasses; ++p) {
    const int r = r0 + p * RPP;
    const bool ok = inside && r < rows;
    o[p] = ok ? *reinterpret_cast<const u32x4*>(O + stat_row_offset(geo, so, hh, r) + sub * 8) : z;
    g[p] = ok ? *reinterpret_cast<const u32x4*>(dO + stat_row_offset(geo, sdo, hh, r) + sub * 8) : z;
  }
#pragma unroll
  for (int p = 0; p < kPrePasses; ++p) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = __builtin_fmaf(T::to_f32((uint16_t)(o[p][w] & 0xffff)), T::to_f32((uint16_t)(g[p][w] & 0xffff)), s);
      s = __builtin_fmaf(T::to_f32((uint16_t)(o[p][w] >> 16)), T::to_f32((uint16_t)(g[p][w] >> 16)), s);
    }
    // every lane takes part (rows past the head reduce zeros), so the shuffles stay in-row
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const int r = r0 + p * RPP;
    if (sub == 0 && r < rows) delta[(long long)hh * rows + r] = s;
  }
}

// ------------------------------------------------------------------------------------------
// [3] dQ. Workgroup = NW waves, each owning 32 query rows (Q, dO, LSE, D pinned); K/V tiles of
// BN keys are copied global -> LDS (swizzled) by the asynchronous loads into a
// double-buffered ring.
//
// Per step and wave, S^T = K Q^T and dP^T = V dO^T put one query row in each lane (its LSE
// and D are per-lane scalars). The step is written as three sched_barrier-fenced phases of
// BN/32 * 8 MFMAs with the LDS fragment reads issued ahead of their MFMA:
//   [S]  S^T = K Q^T          || the copies of the next K / V tile
//   [dP] dP^T = V dO^T        || P = 2^(c S - LSE log2 e)
//   [dQ] dQ^T += K^T dS^T     || dS = P (dP - D) of the next 16-key group
// Steps on the causal diagonal or the key tail run a copy of the body with the mask.
template <typename T, int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, D <= 128 ? 2 : 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dQ, Geom geo, Strides sq, Strides sk, Strides sv, Strides sdo, Strides sdq,
    int n_qtiles_max, int pair, float scale, float c_log2, const uint16_t* __restrict__ O, Strides so,
    float* __restrict__ DeltaOut) {
  constexpr int KB = BN / 32;  // 32-key blocks per K/V tile
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPW = BN * D * 2 / 1024 / NW;  // tile copies per wave per K (or V) tile
  static_assert(CPW >= 1, "each wave copies at least one KB of a tile");

  // K is read by rows (S^T) and transposed (dQ), V by rows: swizzled layout for both.
  // One array per ring slot: with every slot index a compile-time constant the compiler can
  // tell a copy into one slot from reads of another and does not wait for the copy first.
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps copy setup scalar
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Causal: when the grid is large (pair), a workgroup takes the pair of Q tiles
  // (n_qtiles-1-p, p), the heavy one first, so every workgroup has the same number of K/V
  // tiles; an odd middle tile runs alone. On a grid too small to fill the CUs twice over, one
  // tile per workgroup, the heaviest first. A head's workgroups run together on one XCD
  // (shared K/V reads in its L2).
  // The grid covers the longest sequence; a workgroup past its own sequence's tiles exits.
  const int BH = geo.B * geo.H;
  const bool paired = CAUSAL && pair != 0;
  const int npairs = paired ? (n_qtiles_max + 1) / 2 : n_qtiles_max;
  const int lid = xcd_local_index(blockIdx.x, BH * npairs);
  // wave-uniform (keeps pointers scalar)
  const int bh = __builtin_amdgcn_readfirstlane(head_of_item(lid / npairs, geo.B, geo.H));
  const int pr = __builtin_amdgcn_readfirstlane(lid % npairs);
  const Seq sq_ = seq_of(geo, bh);
  const int N = sq_.n;    // query rows of this sequence
  const int NK = sq_.nk;  // key rows
  const int off = NK - N;  // causal: query i sees key j iff j <= i + off
  const int n_qtiles = (N + BM - 1) / BM;
  if (pr >= (paired ? (n_qtiles + 1) / 2 : n_qtiles)) return;
  const int npass = (paired && n_qtiles - 1 - pr != pr) ? 2 : 1;
  const uint16_t* Qh = seq_base(Q, sq, sq_);
  const uint16_t* Kh = seq_base_k(K, sk, sq_);
  const uint16_t* Vh = seq_base_k(V, sv, sq_);
  const uint16_t* dOh = seq_base(dO, sdo, sq_);
  uint16_t* dQh = seq_base(dQ, sdq, sq_);
  const int rsq = (int)sq.r, rsk = (int)sk.r, rsv = (int)sv.r, rsdo = (int)sdo.r, rsdq = (int)sdq.r;
  for (int pass = 0; pass < npass; ++pass) {
  const int qt = CAUSAL ? (pass == 0 ? n_qtiles - 1 - pr : pr) : pr;
  // every wave is done with the previous tile's LDS slots before this tile's copies start
  if (pass > 0) __syncthreads();
  const int q0 = qt * BM;
  const int qrow = q0 + wave * 32 + l32;  // this lane's query row

  // Keys [0, kv_end) are visible to some row of the workgroup (none: dQ = 0).
  const int kv_end = CAUSAL ? min(NK, max(0, q0 + BM + off)) : NK;
  const int ntiles = (kv_end + BN - 1) / BN;
  // Tiles [0, n_plain) have every key visible to every row of the workgroup: no mask.
  const int n_plain = CAUSAL ? min(NK, max(0, q0 + off + 1)) / BN : NK / BN;
  // Keys past NK, and with the causal mask keys after row + off, are hidden: key <= key_lim.
  const int key_lim = CAUSAL ? min(qrow + off, NK - 1) : NK - 1;

  const int dh = geo.dh;
  stage_rows_swz_buf<D, BN, NW>(lds_k0, Kh, 0, NK, rsk, dh, wave);
  stage_rows_swz_buf<D, BN, NW>(lds_v0, Vh, 0, NK, rsv, dh, wave);

  Frag qf[KS], dof[KS];
  float lse2, dl;
  {
    const bool ok = qrow < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool okc = ok && ks * 16 + h * 8 < dh;
      qf[ks].v = gload16(Qh + (size_t)qrow * rsq + ks * 16 + h * 8, okc);
      dof[ks].v = gload16(dOh + (size_t)qrow * rsdo + ks * 16 + h * 8, okc);
    }
    lse2 = ok ? LSE[sq_.stat + qrow] * kLog2e : 0.f;
    if (O != nullptr) {
      // With O given, this workgroup computes D for its own rows in place of the preprocess
      // stage, by the same definition (D_i = sum_c dO_ic O_ic from the stored O, fp32): the
      // lane's half of the row (the columns of its dO fragments), then its partner lane's half,
      // and writes it for the dK/dV stage.
      const uint16_t* Oh = seq_base(O, so, sq_);
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ov = gload16(Oh + (size_t)qrow * so.r + ks * 16 + h * 8, ok && ks * 16 + h * 8 < dh);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t g = dof[ks].v[w];
          part = __builtin_fmaf(T::to_f32((uint16_t)(ov[w] & 0xffff)), T::to_f32((uint16_t)(g & 0xffff)), part);
          part = __builtin_fmaf(T::to_f32((uint16_t)(ov[w] >> 16)), T::to_f32((uint16_t)(g >> 16)), part);
        }
      }
      dl = half_swap_sum(part);
      if (ok && h == 0) DeltaOut[sq_.stat + qrow] = dl;
    } else {
      dl = ok ? Delta[sq_.stat + qrow] : 0.f;
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // Loop-invariant per-lane byte offsets of every fragment read (the swizzle is linear over
  // XOR): K / V row reads need one offset per k-step, K^T transposing reads two per 32-column
  // block; row steps are adds folded into the instructions.
  int rofs[KS], cofs[DB][2];
  {
    const int r0 = swz_rows_base<D>(0) * 2, c0 = swz_cols_base<D>() * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rofs[ks] = r0 ^ (ks << 5);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      cofs[db][0] = c0 ^ (db << 6);
      cofs[db][1] = cofs[db][0] ^ 32;
    }
  }
  auto tfrag = [&](const uint16_t* tile, int db, int krow0) __attribute__((always_inline)) {
    return lds_read_cols(tile, cofs[db][0] + krow0 * D * 2, cofs[db][1] + (krow0 + 8) * D * 2);
  };

  wait_async();
  __syncthreads();

  // One K/V tile: reads slots (kc, vc) holding tile t, copies tile t+1 (clamped: the
  // prefetch is unconditional) into (kn, vn). Register i of S^T / dP^T holds key
  // t*BN + 8(i/4) + 4h + (i%4) of this lane's query row.
  auto step = [&](auto mask_tag, int t, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn)
                  __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int NA = KB * KS;  // MFMAs of the [S] and of the [dP] phase
    // Register r of key block b holds key t*BN + 4h + b*32 + 8(r/4) + (r%4); it is visible to
    // this lane's row iff key <= key_lim, i.e. iff its compile-time offset is <= thr.
    const int thr = key_lim - t * BN - 4 * h;
    const int tn = min(t + 1, ntiles - 1);
    const TileSrc rk = tile_src<D, BN>(Kh, tn * BN, NK, rsk, dh);
    const TileSrc rv = tile_src<D, BN>(Vh, tn * BN, NK, rsv, dh);
    // fragment i of a K or V tile: key block i % KB (so consecutive MFMAs are independent),
    // k-step i / KB
    auto rfrag = [&](const uint16_t* tile, int i) {
      return lds_read_rows(tile, rofs[i / KB] + (i % KB) * 32 * D * 2);
    };

    // ---- [S]: chunk i issues a tile copy every GAP chunks, the K fragment read for MFMA i+2
    // and MFMA i.
    f32x16 s[KB], dp[KB];
    {
      constexpr int GAP = NA / (2 * CPW);
      static_assert(GAP >= 1 && NA % (2 * CPW) == 0, "copies must spread evenly over [S]");
      Frag fr[3];
      fr[0] = rfrag(kc, 0);
      fr[1] = rfrag(kc, 1);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i % GAP == 0) {
          const int c = i / GAP;
          if (c < CPW)
            stage_copy<D, BN, NW>(kn, rk, wave, c);
          else
            stage_copy<D, BN, NW>(vn, rv, wave, c - CPW);
        }
        if (i + 2 < NA) fr[(i + 2) % 3] = rfrag(kc, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = i % KB, ks = i / KB;
        s[kb] = T::mfma(fr[i % 3], qf[ks], ks == 0 ? f32x16{} : s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- [dP]: chunk i issues the V fragment read for MFMA i+2, MFMA i and 16/KS
    // exponentials of S.
    {
      constexpr int EPC = 16 * KB / NA;
      Frag fr[3];
      fr[0] = rfrag(vc, 0);
      fr[1] = rfrag(vc, 1);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + 2 < NA) fr[(i + 2) % 3] = rfrag(vc, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = i % KB, ks = i / KB;
        dp[kb] = T::mfma(fr[i % 3], dof[ks], ks == 0 ? f32x16{} : dp[kb]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int idx = i * EPC + e, b = idx / 16, r = idx % 16;
          float x = __builtin_fmaf(s[b][r], c_log2, -lse2);
          if (MASK) {
            // hidden entries get 2^-inf = 0: a select on the exponent input when the
            // element's compile-time key offset exceeds the lane's threshold
            x = (b * 32 + 8 * (r / 4) + (r % 4)) > thr ? -INFINITY : x;
          }
          s[b][r] = __builtin_amdgcn_exp2f(x);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- dS = P (dP - D) of the first 16-key group, then [dQ]: chunk j (group g = j / DB,
    // keys 16g .. 16g+15 of the tile, d block db = j % DB) issues the K^T fragment read for
    // MFMA j+1, MFMA j, and during group g's MFMAs dS of group g+1.
    {
      constexpr int NG = 2 * KB;   // 16-key groups
      constexpr int NJ = NG * DB;
      constexpr int EPC = 8 / DB;  // next-group elements per chunk
      Frag dsf[NG];
      Frag fr[2];
      fr[0] = tfrag(kc, 0, 0);
#pragma unroll
      for (int r = 0; r < 8; ++r) dp[0][r] = s[0][r] * (dp[0][r] - dl);
      dsf[0] = pack_group<T>(dp[0], 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int g = j / DB, db = j % DB;
        if (j + 1 < NJ) fr[(j + 1) % 2] = tfrag(kc, (j + 1) % DB, ((j + 1) / DB) * 16);
        __builtin_amdgcn_sched_barrier(0);
        acc[db] = T::mfma(fr[j % 2], dsf[g], acc[db]);
        if (g + 1 < NG) {
          const int gn = g + 1, b = gn / 2;
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const int r = 8 * (gn % 2) + db * EPC + e;
            dp[b][r] = s[b][r] * (dp[b][r] - dl);
            if (r % 2 == 1) dsf[gn].v[(r % 8) / 2] = T::pack2(dp[b][r - 1], dp[b][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Tile t+1 must have landed before anyone reads it.
    wait_async();
    ring_barrier();
  };

  // Two steps per trip with the slots fixed at compile time; the masked loop takes the
  // causal diagonal and the key tail, with one fully masked padding step (its keys are past
  // the causal range or past N) when the count is odd.
  using F = std::false_type;
  using Tr = std::true_type;
  auto pair = [&](auto mask_tag, int t) __attribute__((always_inline)) {
    step(mask_tag, t, lds_k0, lds_v0, lds_k1, lds_v1);
    step(mask_tag, t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  };
  int t = 0;
  for (; t + 2 <= n_plain; t += 2) pair(F(), t);
  for (; t < ntiles; t += 2) pair(Tr(), t);
  // No copy may still be landing in LDS when the workgroup retires.
  wait_async();

  if (qrow < N) {
    uint16_t* row = dQh + (size_t)qrow * rsdq;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack2(acc[db][4 * g + 0] * scale, acc[db][4 * g + 1] * scale);
        w[1] = T::pack2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
        // columns db*32 + 8g + 4h .. +3 exist iff db*32 + 8g < dh (dh is a multiple of 8)
        if (db * 32 + 8 * g < dh) *reinterpret_cast<u32x2*>(row + db * 32 + 8 * g + 4 * h) = w;
      }
  }
  }  // pass
}

// ------------------------------------------------------------------------------------------
// Launchers.

template <typename T, int D>
static hipError_t launch_pre_t(const BwdArgs& a) {
  constexpr int RPB = pre_rows_per_block<D>();
  const int nrb = (stat_rows(a.g) + RPB - 1) / RPB;
  const long long blocks = (long long)stat_heads(a.g) * nrb;
  if (blocks == 0) return hipSuccess;
  return launch_kernel(&bwd_preprocess_kernel<T, D>, (unsigned)blocks, 256, a.stream, (const uint16_t*)a.o,
                       (const uint16_t*)a.dO, a.delta, a.g, a.so, a.sdo, nrb);
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a) {
  constexpr int NW = 4, BN = 64;
  constexpr int BM = NW * 32;
  const int n_qtiles = (a.g.N + BM - 1) / BM;
  const long long BH = (long long)a.g.B * a.g.H;
  const bool pair = CAUSAL && pair_causal_tiles((long long)((n_qtiles + 1) / 2) * BH);
  const long long grid = (pair ? (n_qtiles + 1) / 2 : n_qtiles) * BH;
  if (grid == 0) return hipSuccess;
  return launch_kernel(&bwd_dq_kernel<T, D, BN, NW, CAUSAL>, (unsigned)grid, NW * 64, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.delta,
                       (uint16_t*)a.dq, a.g, a.sq, a.sk, a.sv, a.sdo, a.sdq, n_qtiles, pair ? 1 : 0, a.scale,
                       a.c_log2, a.dq_delta ? (const uint16_t*)a.o : nullptr, a.so,
                       a.dq_delta ? a.delta : nullptr);
}

template <typename T>
static hipError_t pre_dt(const BwdArgs& a) {
  return a.d <= 64 ? launch_pre_t<T, 64>(a) : a.d <= 128 ? launch_pre_t<T, 128>(a) : launch_pre_t<T, 256>(a);
}
template <typename T>
static hipError_t dq_dt(const BwdArgs& a) {
  if (a.d <= 64) return a.causal ? launch_dq_t<T, 64, true>(a) : launch_dq_t<T, 64, false>(a);
  if (a.d <= 128) return a.causal ? launch_dq_t<T, 128, true>(a) : launch_dq_t<T, 128, false>(a);
  return a.causal ? launch_dq_t<T, 256, true>(a) : launch_dq_t<T, 256, false>(a);
}

hipError_t launch_bwd_preprocess(const BwdArgs& a) { return a.bf16 ? pre_dt<BF16>(a) : pre_dt<FP16>(a); }
hipError_t launch_bwd_dq(const BwdArgs& a) { return a.bf16 ? dq_dt<BF16>(a) : dq_dt<FP16>(a); }

}  // namespace fa
