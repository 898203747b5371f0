// Exact tiled attention backward, stage [2]: dK and dV ("Triton 05: Flash Attention",
// sections "3단계 커널 구조" and "dKV 커널 수식": K_j and V_j stay on chip while every Q tile i
// streams past; each workgroup owns its dK_j, dV_j, so no atomics are needed).
//
// Per 32-query step and wave (32 keys): S = Q K^T and dP = dO V^T on the matrix cores
// (A = Q / dO rows from LDS, B = the wave's pinned K / its V rows from LDS),
// P = 2^(c*S - LSE*log2 e) with the causal / tail mask folded into the exponent input,
// dS = P * (dP - D), then dV^T += dO^T P and dK^T += Q^T dS (A = transposing LDS reads,
// B = P / dS rounded to the input type). dK is scaled once at the end.
//
// Instruction schedule of a step (one wave; 32 MFMAs in four phases of 8, each phase written
// as sched_barrier-fenced chunks with the LDS fragment reads issued ahead of their MFMA):
//   [S]  8 MFMAs S = Q K^T          || the copies of the next Q / dO tile
//   [dP] 8 MFMAs dP = dO V^T        || P = 2^(c S - LSE log2 e) and its 16-bit packing
//   [dV] 8 MFMAs dV^T += dO^T P     || dS = P (dP - D) and its packing
//   [dK] 8 MFMAs dK^T += Q^T dS
// Steps on the causal diagonal or a tail (queries past N, keys past N) run a copy of the
// body with the mask; all others run without it.
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
__global__ __launch_bounds__(NW * 64, D <= 128 ? 2 : 1) void bwd_dkv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, Geom geo, Strides sq, Strides sk, Strides sv,
    Strides sdo, Strides sdk, Strides sdv, int n_ktiles_max, int pair, float scale, float c_log2) {
  constexpr int BK = NW * 32;
  constexpr int BQ = 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPW = BQ * D * 2 / 1024 / NW;  // tile copies per wave per Q (or dO) tile
  static_assert(CPW >= 1, "each wave copies at least one KB of a tile");
  // d <= 64: D folded into the dP product. The wave's V rows are negated once in LDS and each
  // step's dP accumulator starts from D, so the product gives D - dP and P (D - dP) = -dS costs
  // one multiply per element instead of a subtract and a multiply; dK then accumulates -dK and
  // is scaled by -scale. (At d = 128 the 16 registers the initial value needs at the start of
  // the dP phase push spills into the loop.)
  constexpr bool DFOLD = D <= 64;

  // The workgroup's V tile stays in LDS; Q/dO tiles stream. All tiles are swizzled (row and
  // transposed reads are both conflict-free). One array per ring slot, every slot index a
  // compile-time constant: the compiler can then tell a copy into one slot from a read of
  // another and does not wait for the copy first.
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_q0[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_q1[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_do0[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_do1[BQ * D];
  __shared__ __attribute__((aligned(512))) float lds_st0[128];  // [0,32): LSE, [kStatB, +32): D
  __shared__ __attribute__((aligned(512))) float lds_st1[128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps copy setup scalar
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Causal: low key tiles see the most queries. When the grid is large (pair), a workgroup
  // takes the pair of key tiles (p, n_ktiles-1-p), the heavy one first, so every workgroup
  // streams the same number of Q tiles; an odd middle tile runs alone. On a grid too small to
  // fill the CUs twice over, one tile per workgroup, the heaviest (p = 0) first. A head's
  // workgroups run together on one XCD (shared Q/dO reads in its L2).
  // The grid covers the longest sequence; a workgroup past its own sequence's tiles exits.
  const int BH = geo.B * geo.H;
  const bool paired = CAUSAL && pair != 0;
  const int npairs = paired ? (n_ktiles_max + 1) / 2 : n_ktiles_max;
  const int lid = xcd_local_index(blockIdx.x, BH * npairs);
  // wave-uniform (keeps pointers scalar)
  const int bh = __builtin_amdgcn_readfirstlane(head_of_item(lid / npairs, geo.B, geo.H));
  const int pr = __builtin_amdgcn_readfirstlane(lid % npairs);
  const Seq sq_ = seq_of(geo, bh);
  const int N = sq_.n;    // query rows of this sequence
  const int NK = sq_.nk;  // key rows
  const int off = NK - N;  // causal: query i sees key j iff j <= i + off
  const int n_ktiles = (NK + BK - 1) / BK;
  if (pr >= (paired ? (n_ktiles + 1) / 2 : n_ktiles)) return;
  const int npass = (paired && n_ktiles - 1 - pr != pr) ? 2 : 1;
  const uint16_t* Qh = seq_base(Q, sq, sq_);
  const uint16_t* Kh = seq_base_k(K, sk, sq_);
  const uint16_t* Vh = seq_base_k(V, sv, sq_);
  const uint16_t* dOh = seq_base(dO, sdo, sq_);
  uint16_t* dKh = seq_base_k(dK, sdk, sq_);
  uint16_t* dVh = seq_base_k(dV, sdv, sq_);
  const int rsq = (int)sq.r, rsk = (int)sk.r, rsv = (int)sv.r, rsdo = (int)sdo.r;
  const float* lse_h = LSE + sq_.stat;
  const float* dl_h = Delta + sq_.stat;
  for (int pass = 0; pass < npass; ++pass) {
  const int kt = pass == 0 ? pr : n_ktiles - 1 - pr;
  // every wave is done with the previous tile's LDS slots before this tile's copies start
  if (pass > 0) __syncthreads();
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;


  // Query steps [it_begin, it_end) hold every query that sees a key of this tile (query i
  // sees key j iff j <= i + off).
  const int it_begin = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int it_end = (N + BQ - 1) / BQ;
  // The steps run downwards, from the end of the sequence to it_begin: every workgroup of a
  // head then starts on the same query rows at about the same time and they share those
  // reads in their XCD's L2, where an upward sweep from each tile's own diagonal would have
  // them at different rows. Steps go in pairs; an odd count starts with one step past N
  // (it_end), fully masked and reading zeros.
  const int it_top = it_begin + ((it_end - it_begin + 1) & ~1) - 1;

  const int dh = geo.dh;
  if (it_begin >= it_end) {
    // No query sees these keys (more keys than queries, causal): dK = dV = 0.
    if (key < NK) {
      uint16_t* dk_row = dKh + (size_t)key * sdk.r;
      uint16_t* dv_row = dVh + (size_t)key * sdv.r;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (db * 32 + 8 * g < dh) {
            *reinterpret_cast<u32x2*>(dk_row + db * 32 + 8 * g + 4 * h) = u32x2{0u, 0u};
            *reinterpret_cast<u32x2*>(dv_row + db * 32 + 8 * g + 4 * h) = u32x2{0u, 0u};
          }
    }
    continue;
  }
  // At two waves per SIMD registers are short: one lane offset serves all of a wave's copies.
  constexpr bool SHARE = D <= 128;
  stage_rows_swz_buf<D, BK, NW, SHARE>(lds_v, Vh, k0, NK, rsv, dh, wave);
  stage_rows_swz_buf<D, BQ, NW, SHARE>(lds_q0, Qh, it_top * BQ, N, rsq, dh, wave);
  stage_rows_swz_buf<D, BQ, NW, SHARE>(lds_do0, dOh, it_top * BQ, N, rsdo, dh, wave);
  if (wave == NW - 1) stage_stats_buf((FA_LDS float*)lds_st0, lse_h, dl_h, it_top * BQ, N);

  // Pinned K fragments (B operand of S = Q K^T): lane holds K[key][16ks + 8h .. +7].
  Frag kf[KS];
  {
    const bool ok = key < NK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks].v = gload16(Kh + (size_t)key * rsk + ks * 16 + h * 8, ok && ks * 16 + h * 8 < dh);
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
  if constexpr (DFOLD) {
    // this wave's V rows, the only ones it reads, sign-flipped in place (exact)
    u32x4* vw = reinterpret_cast<u32x4*>(lds_v + wave * 32 * D);
#pragma unroll
    for (int c = 0; c < 32 * D * 2 / 16 / 64; ++c) {
      u32x4 x = vw[c * 64 + lane];
      x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      vw[c * 64 + lane] = x;
    }
  }

  // Loop-invariant per-lane byte offsets of every fragment read (the swizzle is linear over
  // XOR): row reads of Q / dO / V need one offset per k-step, transposing reads of Q / dO two
  // per 32-column block; tile bases and row steps are adds folded into the instructions.
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
  // Transposing fragment: rows krow0 .. krow0 + 15 (k index), columns of d block db.
  auto tfrag = [&](const uint16_t* tile, int db, int krow0) __attribute__((always_inline)) {
    return lds_read_cols(tile, cofs[db][0] + krow0 * D * 2, cofs[db][1] + (krow0 + 8) * D * 2);
  };

  // One 32-query step: reads slot (qs, dos, st), copies the next tile into (qn, don, stn).
  // Register i of S / dP holds query row qbase + 8(i/4) + 4h + (i%4) and this lane's key.
  // (always_inline: six copies of this body exceed the inliner's budget, and a call would
  // leave the accumulators in scratch memory)
  auto step = [&](auto mask_tag, int it, const uint16_t* qs, const uint16_t* dos, const float* st, uint16_t* qn,
                  uint16_t* don, FA_LDS float* stn) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int qbase = it * BQ;
    // Register i holds query row qbase + 4h + 8(i/4) + (i%4) of this lane's key. It is visible
    // iff the row is < N, the key is < NK and (causal) row + off >= key, i.e. iff the
    // compile-time offset 8(i/4) + (i%4) lies in [vis_lo, vis_hi); one unsigned compare.
    const int vis_lo = CAUSAL ? key - off - qbase - 4 * h : -(1 << 24);
    const int vis_hi = key < NK ? N - qbase - 4 * h : vis_lo;
    const uint32_t vis_span = (uint32_t)max(vis_hi - vis_lo, 0);
    // this wave's V rows: base offset re-materialised each step (kept opaque so the compiler
    // adds it per read instead of holding KS more loop-invariant addresses)
    int vrow = wave * 32 * D * 2;
    asm volatile("" : "+v"(vrow));
    const int itn = max(it - 1, it_begin);  // the next step's tile (clamped: the copy is unconditional)
    const TileSrc rq = tile_src<D, BQ>(Qh, itn * BQ, N, rsq, dh);
    const TileSrc rdo = tile_src<D, BQ>(dOh, itn * BQ, N, rsdo, dh);
    if (wave == NW - 1) stage_stats_buf(stn, lse_h, dl_h, itn * BQ, N);

    // this lane's LSE (then D) values for register group g (rows 8g + 4h .. +3), each read
    // one group ahead of its use inside the chunks below
    f32x4 st4[4];
    auto st_read = [&](int base, int g) { return *reinterpret_cast<const f32x4*>(&st[base + 8 * g + 4 * h]); };
    st4[0] = st_read(0, 0);

    // ---- [S]: chunk ks issues a tile copy every GAP chunks, the Q fragment read for MFMA
    // ks+2 and MFMA ks.
    f32x16 s, dp;
    {
      constexpr int GAP = KS / (2 * CPW);
      static_assert(GAP >= 1 && KS % (2 * CPW) == 0, "copies must spread evenly over [S]");
      Frag qfr[3];
      qfr[0] = lds_read_rows(qs, rofs[0]);
      qfr[1] = lds_read_rows(qs, rofs[1]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks % GAP == 0) {
          const int c = ks / GAP;
          if (c < CPW)
            stage_copy<D, BQ, NW, SHARE>(qn, rq, wave, c);
          else
            stage_copy<D, BQ, NW, SHARE>(don, rdo, wave, c - CPW);
        }
        if (ks + 2 < KS) qfr[(ks + 2) % 3] = lds_read_rows(qs, rofs[ks + 2]);
        __builtin_amdgcn_sched_barrier(0);
        s = T::mfma(qfr[ks % 3], kf[ks], ks == 0 ? f32x16{} : s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- [dP]: chunk ks issues the dO and V fragment reads for MFMA ks+1, MFMA ks, and the
    // exponentials (and packing) of 16/KS scores of S.
    Frag pf[2], df[2];
    {
      constexpr int EPC = 16 / KS;  // elements per chunk
      Frag dfr[2], vfr[2];
      f32x16 dini;  // DFOLD: D of register i's row, the dP accumulator's initial value
      if constexpr (DFOLD) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 d4 = st_read(kStatB, g);
#pragma unroll
          for (int e = 0; e < 4; ++e) dini[4 * g + e] = d4[e];
        }
      }
      dfr[0] = lds_read_rows(dos, rofs[0]);
      vfr[0] = lds_read_rows(lds_v, rofs[0] + vrow);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          dfr[(ks + 1) % 2] = lds_read_rows(dos, rofs[ks + 1]);
          vfr[(ks + 1) % 2] = lds_read_rows(lds_v, rofs[ks + 1] + vrow);
        }
        if ((ks * EPC) % 4 == 0 && (ks * EPC) / 4 + 1 < 4) st4[(ks * EPC) / 4 + 1] = st_read(0, (ks * EPC) / 4 + 1);
        if (!DFOLD && ks == KS - 1) st4[0] = st_read(kStatB, 0);
        __builtin_amdgcn_sched_barrier(0);
        dp = T::mfma(dfr[ks % 2], vfr[ks % 2], ks == 0 ? (DFOLD ? dini : f32x16{}) : dp);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int i = ks * EPC + e;
          float x = __builtin_fmaf(s[i], c_log2, -st4[i / 4][i % 4] * kLog2e);
          if (MASK) {
            // hidden entries get 2^-inf = 0: a select on the exponent input unless the
            // element's compile-time row offset lies in [vis_lo, vis_lo + vis_span)
            x = (uint32_t)(8 * (i / 4) + (i % 4) - vis_lo) >= vis_span ? -INFINITY : x;
          }
          s[i] = __builtin_amdgcn_exp2f(x);
          if (i % 2 == 1) pf[i / 8].v[(i % 8) / 2] = T::pack2(s[i - 1], s[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- [dV]: chunk j (16-key half tt = j / DB, d block db = j % DB) issues the dO^T
    // fragment read for MFMA j+1, MFMA j, and dS (and packing) of 16/(2 DB) elements.
    {
      constexpr int NJ = 2 * DB;
      constexpr int EPC = 16 / NJ;
      Frag tfr[2];
      tfr[0] = tfrag(dos, 0, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j + 1 < NJ) tfr[(j + 1) % 2] = tfrag(dos, (j + 1) % DB, ((j + 1) / DB) * 16);
        if (!DFOLD && (j * EPC) % 4 == 0 && (j * EPC) / 4 + 1 < 4)
          st4[(j * EPC) / 4 + 1] = st_read(kStatB, (j * EPC) / 4 + 1);
        __builtin_amdgcn_sched_barrier(0);
        acc_dv[j % DB] = T::mfma(tfr[j % 2], pf[j / DB], acc_dv[j % DB]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int i = j * EPC + e;
          dp[i] = DFOLD ? s[i] * dp[i] : s[i] * (dp[i] - st4[i / 4][i % 4]);  // DFOLD: -dS
          if (i % 2 == 1) df[i / 8].v[(i % 8) / 2] = T::pack2(dp[i - 1], dp[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- [dK]: chunk j issues the Q^T fragment read for MFMA j+1 and MFMA j.
    {
      constexpr int NJ = 2 * DB;
      Frag tfr[2];
      tfr[0] = tfrag(qs, 0, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j + 1 < NJ) tfr[(j + 1) % 2] = tfrag(qs, (j + 1) % DB, ((j + 1) / DB) * 16);
        __builtin_amdgcn_sched_barrier(0);
        acc_dk[j % DB] = T::mfma(tfr[j % 2], df[j / DB], acc_dk[j % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // The next tile must have landed before anyone reads it.
    wait_async();
    ring_barrier();
  };

  // Two steps per trip (it, then it - 1) with the slots fixed at compile time. Masked steps:
  // the partial query tile at the top (and the padding step), every step when this tile has
  // keys past NK, and the causal diagonal at the bottom; the plain loop takes the full query
  // tiles in between.
  using F = std::false_type;
  using Tr = std::true_type;
  auto pair = [&](auto mask_tag, int it) __attribute__((always_inline)) {
    step(mask_tag, it, lds_q0, lds_do0, lds_st0, lds_q1, lds_do1, (FA_LDS float*)lds_st1);
    step(mask_tag, it - 1, lds_q1, lds_do1, lds_st1, lds_q0, lds_do0, (FA_LDS float*)lds_st0);
  };
  const bool key_tail = k0 + BK > NK;
  // the first step whose rows all see every key of the tile: qbase + off >= k0 + BK - 1
  const int full_from = max(0, k0 + BK - 1 - off);
  const int plain_begin = key_tail ? it_end : (CAUSAL ? min(it_end, max(it_begin, (full_from + BQ - 1) / BQ)) : it_begin);
  const int plain_end = key_tail ? it_end : max(plain_begin, N / BQ);
  int it = it_top;
  for (; it >= plain_end; it -= 2) pair(Tr(), it);
  for (; it - 1 >= plain_begin; it -= 2) pair(F(), it);
  for (; it > it_begin; it -= 2) pair(Tr(), it);
  // No copy may still be landing in LDS when the workgroup retires.
  wait_async();

  if (key < NK) {
    uint16_t* dk_row = dKh + (size_t)key * sdk.r;
    uint16_t* dv_row = dVh + (size_t)key * sdv.r;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk, wv;
        constexpr float sgn = DFOLD ? -1.f : 1.f;  // DFOLD: acc_dk holds -dK / scale
        wk[0] = T::pack2(acc_dk[db][4 * g + 0] * (sgn * scale), acc_dk[db][4 * g + 1] * (sgn * scale));
        wk[1] = T::pack2(acc_dk[db][4 * g + 2] * (sgn * scale), acc_dk[db][4 * g + 3] * (sgn * scale));
        wv[0] = T::pack2(acc_dv[db][4 * g + 0], acc_dv[db][4 * g + 1]);
        wv[1] = T::pack2(acc_dv[db][4 * g + 2], acc_dv[db][4 * g + 3]);
        // columns db*32 + 8g + 4h .. +3 exist iff db*32 + 8g < dh (dh is a multiple of 8): a
        // wave-uniform test
        if (db * 32 + 8 * g < dh) {
          *reinterpret_cast<u32x2*>(dk_row + db * 32 + 8 * g + 4 * h) = wk;
          *reinterpret_cast<u32x2*>(dv_row + db * 32 + 8 * g + 4 * h) = wv;
        }
      }
  }
  }  // pass
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_dkv_t(const BwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BK = NW * 32;
  const int n_ktiles = (a.g.Nk + BK - 1) / BK;
  const long long BH = (long long)a.g.B * a.g.H;
  const bool pair = CAUSAL && pair_causal_tiles((long long)((n_ktiles + 1) / 2) * BH);
  const long long grid = (pair ? (n_ktiles + 1) / 2 : n_ktiles) * BH;
  if (grid == 0) return hipSuccess;
  return launch_kernel(&bwd_dkv_kernel<T, D, NW, CAUSAL>, (unsigned)grid, NW * 64, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.delta,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, a.g, a.sq, a.sk, a.sv, a.sdo, a.sdk, a.sdv, n_ktiles,
                       pair ? 1 : 0, a.scale, a.c_log2);
}

#ifndef FA_DKV_WIDE_UNIT
template <typename T>
static hipError_t dkv_dt(const BwdArgs& a) {
  if (a.d <= 64) return a.causal ? launch_dkv_t<T, 64, true>(a) : launch_dkv_t<T, 64, false>(a);
  if (a.d <= 128) return a.causal ? launch_dkv_t<T, 128, true>(a) : launch_dkv_t<T, 128, false>(a);
  return launch_bwd_dkv_wide(a);
}

hipError_t launch_bwd_dkv(const BwdArgs& a) { return a.bf16 ? dkv_dt<BF16>(a) : dkv_dt<FP16>(a); }
#else
// The 256-wide instances (head dims above 128), built in their own unit (fa_bwd_dkv_wide.hip).
hipError_t launch_bwd_dkv_wide(const BwdArgs& a) {
  if (a.bf16) return a.causal ? launch_dkv_t<BF16, 256, true>(a) : launch_dkv_t<BF16, 256, false>(a);
  return a.causal ? launch_dkv_t<FP16, 256, true>(a) : launch_dkv_t<FP16, 256, false>(a);
}
#endif

}  // namespace fa
