// Exact tiled attention forward for gfx950 (CDNA4).
//
// What it computes: O = softmax(scale * Q K^T, optional causal mask) V and the natural-log
// row LSE, never writing S or P anywhere ("Triton 05: Flash Attention", sections
// "Online Softmax", "코드 라인별 설명 (Forward)", "최종 정규화"; "GPU에서 Attention은 실제로
// 어떻게 실행되는가", sections 2-1..2-3 and 3-2).
//
// Work split (Q-outer, as in the FA2 walk-through, section 2-1): one workgroup per
// (batch*head, Q tile of BM = 32*NW rows); each of its NW waves owns 32 whole query rows
// ("split-Q", section 2-3), so row statistics never leave the wave. K/V tiles of BN keys are
// copied global -> LDS by the asynchronous loads (no VGPR round trip) into swizzled ring slots.
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
//
// Software pipeline (one wave's instruction stream; both halves of a step are independent):
//   step t:  [A] S(t+1) = K(t+1) Q^T (matrix cores)   ||  P(t) = 2^(c S(t) - m), row sums (VALU)
//            [B] O^T += V(t)^T P(t)    (matrix cores)  ||  mask + row max of S(t+1)     (VALU)
// so the exponentials of one tile run while the matrix cores compute the next tile's scores,
// and the max reduction runs under the P V products. The ring staggers K one tile ahead of
// V: step t reads K(t+1) and V(t) while the copies of K(t+2) and V(t+1) land in the slots
// that held K(t) and V(t-1); one barrier per step publishes them. At d <= 64 (a short step)
// the ring has three slots each and the copies one step more to land: step t copies K(t+3)
// and V(t+2), and its barrier waits only for the previous step's copies.
//
// Two-group ping-pong (NW = 8, 128-wide tiles, a separate entry point): the matrix product of
// one query sub-tile runs while the softmax of another runs ("FlashAttention·FA4·FP4", section
// "HBM을 아낀 뒤에는 무엇이 기다리는가"; "Triton 05", section "4. H100, B200에서의 추가 기법").
// A workgroup holds 256 query rows in two groups of four waves; the waves of both groups share
// the SIMDs pairwise, and group Y runs half a step behind group X, with a workgroup barrier
// after every half step, so each SIMD pairs one wave's [A] half (exponentials) with the other's
// [B] half (products). The default four-wave form leaves that pairing to the hardware, which
// interleaves the waves of two independent workgroups on each SIMD.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

#include <type_traits>

namespace fa {

// Largest tolerated excess of a tile's max over the reference max, in log2 units: p <= 2^8.
constexpr float kTau = 8.0f;

// SPLIT: the split-KV form ("FlashAttentionを1から", section "その後の版と、推論での事情":
// partial softmax states over disjoint key ranges merge exactly). The key tiles of
// each Q tile are cut into `splits` contiguous ranges, one workgroup each; instead of O and
// LSE a workgroup writes its unnormalised fp32 accumulator, its reference max (log2 units,
// -inf for a row that saw no key) and its row sum to `part`, laid out as
// [splits][BH*N][D] accumulators, then [splits][BH*N] maxima, then [splits][BH*N] sums;
// merge_kernel combines them.
template <typename T, int D, int BN, int NW, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NW * 64, (D <= 64 && NW == 4 && (SPLIT || !CAUSAL)) ? 3 : (D <= 128 && NW == 4) ? 2 : 1) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, Geom geo, Strides sq, Strides sk, Strides sv, Strides so,
    int n_qtiles_max, int pair, float c_log2, float* __restrict__ part, long long rows_all, int splits) {
  constexpr int BM = NW * 32;  // query rows per workgroup
  constexpr int KS = D / 16;   // k-steps over the head dim
  constexpr int DB = D / 32;   // 32-wide blocks of the head dim
  constexpr int KB = BN / 32;  // 32-key blocks per tile
  constexpr int NE = 16 * KB;  // scores of a tile per lane
  static_assert(KB == 2, "the instruction interleaving below is laid out for 64-key tiles");
  // fp16 at d <= 64: the row sum l comes from the matrix cores, in place of 32 VALU adds per
  // step (at this head dim the VALU, not the matrix cores, bounds the step). Each 16-key group
  // of P, already packed as the B operand of the P V product, is also the B operand of one
  // 16x16x32 product whose A operand selects, for each output row, the lanes that hold one
  // query's keys: with B read in that instruction's layout (lane l: column l%16, k = 8(l/16)+j),
  // A[m][k] = 1 iff (m/4) and (k/8) have the same parity, and lane l's first result register
  // (row 4(l/16)) is the sum of its own query's 16 keys. The sum is over P rounded to fp16
  // (relative error at most 2^-11 in l), so O = sum p v / sum p is normalised by exactly the
  // weights its product used.
  constexpr bool MSUM = std::is_same<T, FP16>::value && D == 64 && NW == 4;

  // One array per ring slot, every slot index a compile-time constant: the compiler can then
  // tell a copy into one slot from a read of another and does not wait for the copy first.
  // RING slots each for K and V: two, or three at d <= 64, where a step is short against the
  // latency of its tile copies and three workgroups still fit a CU's LDS (48 KB each).
  constexpr int RING = (D <= 64 && NW == 4) ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k2[RING == 3 ? BN * D : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v2[RING == 3 ? BN * D : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps copy setup scalar
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Causal, when the grid is large (pair): a workgroup takes the pair of Q tiles
  // (n_qtiles-1-p, p), the heavy one first, so every workgroup has the same number of K/V tiles
  // (no tail of long-running workgroups at the end of the grid); an odd middle tile runs alone.
  // On a grid too small to fill the CUs twice over, one tile per workgroup, the heaviest first:
  // the longest workgroup is then one heavy tile instead of a heavy and a light one. A head's
  // workgroups run together on one XCD (shared K/V reads in its L2).
  // Split-KV: one workgroup per (head, Q tile, key range), no pairing.
  // The grid covers the longest sequence; a workgroup past its own sequence's tiles exits.
  const int BH = geo.B * geo.H;
  const bool paired = !SPLIT && CAUSAL && pair != 0;
  const int npairs = SPLIT ? n_qtiles_max * splits : (paired ? (n_qtiles_max + 1) / 2 : n_qtiles_max);
  const int lid = xcd_local_index(blockIdx.x, BH * npairs);
  // wave-uniform (keeps pointers scalar)
  const int bh = __builtin_amdgcn_readfirstlane(head_of_item(lid / npairs, geo.B, geo.H));
  const int pr = __builtin_amdgcn_readfirstlane(lid % npairs);
  const Seq sq_ = seq_of(geo, bh);
  const int N = sq_.n;    // query rows of this sequence
  const int NK = sq_.nk;  // key rows
  const int off = NK - N;  // causal: query i sees key j iff j <= i + off
  const int n_qtiles = (N + BM - 1) / BM;
  const int sp = SPLIT ? pr % splits : 0;  // key range of this workgroup
  if (SPLIT ? pr / splits >= n_qtiles : pr >= (paired ? (n_qtiles + 1) / 2 : n_qtiles)) return;
  const int npass = (paired && n_qtiles - 1 - pr != pr) ? 2 : 1;
  const uint16_t* Qh = seq_base(Q, sq, sq_);
  const uint16_t* Kh = seq_base_k(K, sk, sq_);
  const uint16_t* Vh = seq_base_k(V, sv, sq_);
  uint16_t* Oh = seq_base(O, so, sq_);
  const int rsq = (int)sq.r, rsk = (int)sk.r, rsv = (int)sv.r, rso = (int)so.r;
  for (int pass = 0; pass < npass; ++pass) {
  // (unpaired causal: one tile per workgroup, the heaviest first)
  const int qt = SPLIT ? pr / splits : (CAUSAL ? (pass == 0 ? n_qtiles - 1 - pr : pr) : pr);
  // every wave is done with the previous tile's LDS slots before this tile's copies start
  if (pass > 0) __syncthreads();
  const int q0 = qt * BM;
  const int qrow = q0 + wave * 32 + l32;  // this lane's query row

  // Keys [0, kv_end) are visible to some row of the workgroup.
  const int kv_end = CAUSAL ? min(NK, max(0, q0 + BM + off)) : NK;
  const int ntiles = (kv_end + BN - 1) / BN;
  // Tiles [0, n_plain) have every key visible to every row of the workgroup: no mask.
  const int n_plain = CAUSAL ? min(NK, max(0, q0 + off + 1)) / BN : NK / BN;
  const int dh = geo.dh;
  if (!SPLIT && ntiles == 0) {
    // No row of this tile sees a key (more queries than keys, causal): O = 0, LSE = -inf.
    if (qrow < N) {
      uint16_t* orow = Oh + (size_t)qrow * rso;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (db * 32 + 8 * g < dh) *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = u32x2{0u, 0u};
      if (LSE != nullptr && h == 0) LSE[sq_.stat + qrow] = -INFINITY;
    }
    continue;
  }
  // This workgroup's key tiles [t0, last]: all of them, or its split's share.
  const int t0 = SPLIT ? (int)((long long)sp * ntiles / splits) : 0;
  const int t1 = SPLIT ? (int)((long long)(sp + 1) * ntiles / splits) : ntiles;
  if (SPLIT && t0 >= t1) {
    // An empty key range (more splits than tiles): a state that the merge weighs with zero.
    if (qrow < N) {
      const size_t r = (size_t)sp * rows_all + sq_.stat + qrow;
      float* po = part + r * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g + 4 * h) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (h == 0) {
        part[(size_t)splits * rows_all * D + r] = -INFINITY;
        part[(size_t)splits * rows_all * (D + 1) + r] = 0.f;
      }
    }
    continue;
  }
  const int last = t1 - 1;

  auto stage_k = [&](int t, uint16_t* dst) { stage_rows_swz_buf<D, BN, NW>(dst, Kh, t * BN, NK, rsk, dh, wave); };
  auto stage_v = [&](int t, uint16_t* dst) { stage_rows_swz_buf<D, BN, NW>(dst, Vh, t * BN, NK, rsv, dh, wave); };
  // Ring slot I of K / V (a compile-time index).
  auto kslot = [&](auto ic) __attribute__((always_inline)) -> uint16_t* {
    constexpr int I = decltype(ic)::value;
    if constexpr (I == 0) return lds_k0;
    else if constexpr (I == 1) return lds_k1;
    else return lds_k2;
  };
  auto vslot = [&](auto ic) __attribute__((always_inline)) -> uint16_t* {
    constexpr int I = decltype(ic)::value;
    if constexpr (I == 0) return lds_v0;
    else if constexpr (I == 1) return lds_v1;
    else return lds_v2;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  stage_k(t0, lds_k0);
  stage_v(t0, lds_v0);
  stage_k(min(t0 + 1, last), lds_k1);
  if constexpr (RING == 3) {
    stage_k(min(t0 + 2, last), kslot(S2()));
    stage_v(min(t0 + 1, last), lds_v1);
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qrow][16ks + 8h .. +7].
  Frag qf[KS];
  {
    const bool ok = qrow < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks].v = gload16(Qh + (size_t)qrow * rsq + ks * 16 + h * 8, ok && ks * 16 + h * 8 < dh);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // Row state. m_run: the reference max (log2 units, -inf before any visible key); m_ref: the
  // same, made finite, used as the exponent offset; l_run: this lane's partial row sum (its 16
  // keys of each 32-key block; the two halves are merged in the epilogue).
  float m_run = -INFINITY, m_ref = 0.f, l_run = 0.f;
  float alpha = 1.f;   // rescale factor owed by acc and l before the pending P is added
  // MSUM: the row sum accumulates in lsum[0] instead (the product writes the same sum to all
  // four registers; only lsum[0] is rescaled and read)
  f32x4 lsum = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag sel;  // this lane's A elements: A[l%16][8(l/16) + j], all 1 (fp16) or all 0
  {
    const uint32_t one2 = (((lane >> 2) ^ (lane >> 4)) & 1) ? 0u : 0x3C003C00u;
    sel.v = u32x4{one2, one2, one2, one2};
  }
  auto rowsum_mfma = [&](const Frag& p) __attribute__((always_inline)) {
    lsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, sel.v), __builtin_bit_cast(f16x8, p.v),
                                                  lsum, 0, 0, 0);
  };
  bool moved = false;  // this lane's reference moved for the pending tile

  // Loop-invariant per-lane byte offsets of every fragment read. The swizzle is linear over
  // XOR, so K row reads need one offset per k-step and V^T transposing reads two per 32-column
  // block; key-block, 16-row and 8-row steps are plain adds folded into the instructions.
  int kofs[KS], vofs[DB][2];
  {
    const int r0 = swz_rows_base<D>(0) * 2, c0 = swz_cols_base<D>() * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kofs[ks] = r0 ^ (ks << 5);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      vofs[db][0] = c0 ^ (db << 6);
      vofs[db][1] = vofs[db][0] ^ 32;
    }
  }
  // K fragment i = (key block i / KS, k-step i % KS); V^T fragment (d block db, keys of the
  // 16-key group g).
  auto kfrag = [&](const uint16_t* ktile, int i) __attribute__((always_inline)) {
    return lds_read_rows(ktile, kofs[i % KS] + (i / KS) * 32 * D * 2);
  };
  auto vfrag = [&](const uint16_t* vtile, int db, int g) __attribute__((always_inline)) {
    return lds_read_cols(vtile, vofs[db][0] + g * 16 * D * 2, vofs[db][1] + (g * 16 + 8) * D * 2);
  };

  // S^T tile (32 keys x 32 rows per block) from a K slot.
  auto qk = [&](const uint16_t* ktile, f32x16 (&s)[KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = T::mfma(kfrag(ktile, kb * KS), qf[0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) s[kb] = T::mfma(kfrag(ktile, kb * KS + ks), qf[ks], s[kb]);
    }
  };
  // Masking. A key is visible to this lane's row iff key <= key_lim: keys past NK are hidden,
  // and with the causal mask so are keys after row + off (key_lim < 0: the row sees no key).
  // Register i of key block kb holds key kbase + 4h + kb*32 + 8(i/4) + (i%4), so with
  // thr = key_lim - kbase - 4h an element is hidden iff the compile-time offset
  // kb*32 + 8(i/4) + (i%4) exceeds thr: one compare and one select per element.
  const int key_lim = CAUSAL ? min(qrow + off, NK - 1) : NK - 1;
  auto mask_thr = [&](int t) { return key_lim - t * BN - 4 * h; };
  auto masked = [](float x, int kb, int i, int thr) {
    return (kb * 32 + 8 * (i >> 2) + (i & 3)) > thr ? -INFINITY : x;
  };
  auto mask = [&](f32x16 (&s)[KB], int t) __attribute__((always_inline)) {
    const int thr = mask_thr(t);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = masked(s[kb][i], kb, i, thr);
  };
  // Tile max (this lane's scores) -> new reference, moved lazily: only when the tile's max
  // exceeds the reference by more than kTau; otherwise p = 2^(c s - m_ref) <= 2^kTau
  // accumulates against the old one. O = acc / l and LSE = ln2 (m_ref + log2 l) hold for any
  // reference that acc and l share, so skipping a move only skips a rescale of acc.
  auto update_ref = [&](float mx) __attribute__((always_inline)) {
    mx = half_swap_max(mx) * c_log2;
    moved = mx > m_run + kTau;
    m_run = moved ? mx : m_run;
    // A row that has seen no visible key keeps m_run = -inf; its reference is 0 then.
    const float ref = (m_run == -INFINITY) ? 0.f : m_run;
    // Once a row has a finite reference it only rises, so m_ref - ref <= 0 and alpha lies in
    // [0, 1]. The one exception is the first move away from the placeholder 0, where the
    // first visible tile's max may lie far below zero: 2^(0 - ref) would overflow to +inf
    // there and turn acc * alpha and l * alpha (both 0) into NaN. acc and l hold nothing yet
    // at that point, so any finite factor is exact; clamping the exponent at 0 gives 1.
    alpha = __builtin_amdgcn_exp2f(fminf(m_ref - ref, 0.f));
    m_ref = ref;
  };
  auto row_max = [&](const f32x16 (&s)[KB]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    update_ref(mx);
  };
  // P = 2^(c s - m_ref) packed to 16-bit B operands; l = alpha l + row sum.
  auto softmax_p = [&](f32x16 (&s)[KB], Frag (&pf)[KB][2]) __attribute__((always_inline)) {
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c_log2, -m_ref));
        s[kb][i] = e;
        if (!MSUM) rs += e;
      }
    if (!MSUM) l_run = __builtin_fmaf(l_run, alpha, rs);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pf[kb][0] = pack_group<T>(s[kb], 0);
      pf[kb][1] = pack_group<T>(s[kb], 1);
    }
  };
  // The rescale is owed by the whole wave when any lane's reference moved (alpha = 1 for the
  // others); the branch is wave-uniform and rarely taken.
  auto rescale = [&]() __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      if (MSUM) lsum[0] *= alpha;
    }
  };
  auto pv = [&](const uint16_t* vtile, const Frag (&pf)[KB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < KB * 2; ++g) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = T::mfma(vfrag(vtile, db, g), pf[g / 2][g % 2], acc[db]);
      if (MSUM) rowsum_mfma(pf[g / 2][g % 2]);
    }
  };

  // ---- prologue: K(0), V(0), K(1) landed; S(0) and its reference.
  wait_async();
  __syncthreads();
  f32x16 s[KB];
  qk(lds_k0, s);
  if (t0 >= n_plain) mask(s, t0);
  row_max(s);
  // Every wave is done with slot k0 before the first step copies K(2) over it.
  ring_barrier();

  // ---- steps t = t0 .. last-1, slot phase P = (t - t0) % RING fixed at compile time.
  // (always_inline throughout: at the 256-wide tile these bodies exceed the inliner's budget,
  // and a call would leave the accumulators in scratch memory)
  auto step = [&](auto mask_tag, auto parity_tag, int t) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(parity_tag)::value;
    const uint16_t* kcur = kslot(std::integral_constant<int, (P + 1) % RING>());  // K(t+1)
    const uint16_t* vcur = vslot(std::integral_constant<int, P>());               // V(t)
    uint16_t* kdst = kslot(std::integral_constant<int, P>());  // K(t+RING) replaces K(t)
    uint16_t* vdst = vslot(std::integral_constant<int, (P + RING - 1) % RING>());  // V(t+RING-1) replaces V(t-1)
    // Copies of K(t+RING) and V(t+RING-1): descriptors now, the copies themselves spread over
    // the chunks of [A] (issued all at once, the workgroup's waves queue behind each other in
    // the texture unit right after the barrier).
    const TileSrc rk = tile_src<D, BN>(Kh, min(t + RING, last) * BN, NK, rsk, dh);
    const TileSrc rv = tile_src<D, BN>(Vh, (RING == 2 ? t + 1 : min(t + 2, last)) * BN, NK, rsv, dh);
    constexpr int CPW = BN * D * 2 / 1024 / NW;  // copies per wave per tile

    // [A] S(t+1) on the matrix cores while the VALU exponentiates S(t). Written out as 16
    // chunks fenced by sched_barrier(0), so the order survives the scheduler: chunk i issues
    // every GAP-th chunk one tile copy, the K fragment read for MFMA i+2, MFMA i (the two key
    // blocks alternate, so consecutive MFMAs are independent), and 2 of the 32 exponentials.
    f32x16 sn[KB];
    {
      constexpr int NA = KB * KS;  // MFMAs in this half
      Frag kf[3];
      auto kread = [&](int i) __attribute__((always_inline)) { return kfrag(kcur, (i % KB) * KS + i / KB); };
      kf[0] = kread(0);
      kf[1] = kread(1);
      constexpr int GAP = NA / (2 * CPW);  // chunks between two copies
      static_assert(GAP >= 1 && NA % (2 * CPW) == 0, "copies must spread evenly over [A]");
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i % GAP == 0) {
          const int c = i / GAP;
          if (c < CPW)
            stage_copy<D, BN, NW>(kdst, rk, wave, c);
          else
            stage_copy<D, BN, NW>(vdst, rv, wave, c - CPW);
        }
        if (i + 2 < NA) kf[(i + 2) % 3] = kread(i + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = i % KB, ks = i / KB;
        sn[kb] = T::mfma(kf[i % 3], qf[ks], ks == 0 ? f32x16{} : sn[kb]);
#pragma unroll
        for (int e = 0; e < 32 / NA; ++e) {
          const int idx = i * (32 / NA) + e;
          s[idx / 16][idx % 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[idx / 16][idx % 16], c_log2, -m_ref));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Pin the exponentials here: otherwise the compiler sinks them below the rescale
      // branch, next to their first use, out of reach of the MFMAs above.
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(s[kb]));
    }

    rescale();

    // [B] O += P(t) V(t) on the matrix cores while the VALU finishes P(t) and reduces S(t+1):
    // chunk j issues the V^T fragment reads for MFMA j+2, MFMA j, 4/DB 16-bit conversions of
    // P (a group of 16 keys is converted while the previous group is in use), 2 adds of the
    // row sum and the masked max over 2 scores of S(t+1). MFMAs run key-group-major, so the 4
    // consecutive ones of a group hit independent accumulators.
    {
      constexpr int NG = KB * 2;  // 16-key groups of P
      constexpr int NB = DB * NG;  // MFMAs in this half
      Frag pf[NG];
      pf[0] = pack_group<T>(s[0], 0);
      Frag vf[3];
      auto vread = [&](int j) __attribute__((always_inline)) { return vfrag(vcur, j % DB, j / DB); };
      vf[0] = vread(0);
      vf[1] = vread(1);
      float mx = -INFINITY, rs = 0.f;
      const int thr = mask_thr(t + 1);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (j + 2 < NB) vf[(j + 2) % 3] = vread(j + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int g = j / DB, db = j % DB;
        acc[db] = T::mfma(vf[j % 3], pf[g], acc[db]);
        if (MSUM && db == DB - 1) rowsum_mfma(pf[g]);
        if (g + 1 < NG) {
          // the next group's 4 packed pairs, PPC of them per chunk (the first 4 chunks of the
          // group when it has more than 4)
          const int gn = g + 1;
          constexpr int PPC = DB >= 4 ? 1 : 4 / DB;
#pragma unroll
          for (int c = 0; c < PPC; ++c) {
            const int w = db * PPC + c;
            if (w < 4) pf[gn].v[w] = T::pack2(s[gn / 2][8 * (gn % 2) + 2 * w], s[gn / 2][8 * (gn % 2) + 2 * w + 1]);
          }
        }
#pragma unroll
        for (int e = 0; e < 32 / NB; ++e) {
          const int idx = j * (32 / NB) + e;
          if (!MSUM) rs += s[idx / 16][idx % 16];
          float x = sn[idx / 16][idx % 16];
          if (MASK) {
            x = masked(x, idx / 16, idx % 16, thr);
            sn[idx / 16][idx % 16] = x;
          }
          mx = fmaxf(mx, x);
        }
        asm volatile("" : "+v"(mx), "+v"(rs));  // keep both running reductions in this chunk
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!MSUM) l_run = __builtin_fmaf(l_run, alpha, rs);
      update_ref(mx);
    }

    // K(t+2) and V(t+1) must have landed before anyone reads them: with two slots they are
    // this step's copies; with three, the previous step's, and this step's may stay in flight
    // (the counter drains in issue order).
    if constexpr (RING == 2)
      wait_async();
    else
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * CPW));  // vmcnt(2 CPW)
    ring_barrier();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = sn[kb];
  };
  // ---- the two halves of a step for the two-group ping-pong (NW == 8): [A] S(t+1) || exp S(t),
  // [B] O += P(t) V(t) || row max of S(t+1), each half issuing its group's share of one tile:
  // X copies K(t+2) in [A] and V(t+1) in [B]; Y copies V(t+1) in [A] and K(t+3) in [B].
  f32x16 sn_pp[KB];
  auto half_a = [&](auto mask_tag, auto parity_tag, int t, bool grpY) __attribute__((always_inline)) {
    constexpr int P = decltype(parity_tag)::value;
    const uint16_t* kcur = P ? lds_k0 : lds_k1;  // K(t+1)
    uint16_t* kdst = P ? lds_k1 : lds_k0;        // K(t+2) replaces K(t)
    uint16_t* vdst = P ? lds_v0 : lds_v1;        // V(t+1) replaces V(t-1)
    const TileSrc rk = tile_src<D, BN>(Kh, min(t + 2, last) * BN, NK, rsk, dh);
    const TileSrc rv = tile_src<D, BN>(Vh, (t + 1) * BN, NK, rsv, dh);
    constexpr int CPW = BN * D * 2 / 1024 / NW;
    constexpr int NA = KB * KS;
    constexpr int GAP = NA / CPW;
    Frag kf[3];
    auto kread = [&](int i) __attribute__((always_inline)) { return kfrag(kcur, (i % KB) * KS + i / KB); };
    kf[0] = kread(0);
    kf[1] = kread(1);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i % GAP == 0) {
        if (grpY)
          stage_copy<D, BN, NW>(vdst, rv, wave, i / GAP);
        else
          stage_copy<D, BN, NW>(kdst, rk, wave, i / GAP);
      }
      if (i + 2 < NA) kf[(i + 2) % 3] = kread(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int kb = i % KB, ks = i / KB;
      sn_pp[kb] = T::mfma(kf[i % 3], qf[ks], ks == 0 ? f32x16{} : sn_pp[kb]);
#pragma unroll
      for (int e = 0; e < NE / NA; ++e) {
        const int idx = i * (NE / NA) + e;
        s[idx / 16][idx % 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[idx / 16][idx % 16], c_log2, -m_ref));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(s[kb]));
    rescale();
  };
  auto half_b = [&](auto mask_tag, auto parity_tag, int t, bool grpY) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(parity_tag)::value;
    const uint16_t* vcur = P ? lds_v1 : lds_v0;  // V(t)
    uint16_t* kcur_w = P ? lds_k0 : lds_k1;      // K(t+3) replaces K(t+1)
    uint16_t* vdst = P ? lds_v0 : lds_v1;        // V(t+1) replaces V(t-1)
    const TileSrc rk = tile_src<D, BN>(Kh, min(t + 3, last) * BN, NK, rsk, dh);
    const TileSrc rv = tile_src<D, BN>(Vh, (t + 1) * BN, NK, rsv, dh);
    constexpr int CPW = BN * D * 2 / 1024 / NW;
    constexpr int NG = KB * 2;
    constexpr int NB = DB * NG;
    constexpr int GAP = NB / CPW;
    Frag pf[NG];
    pf[0] = pack_group<T>(s[0], 0);
    Frag vf[3];
    auto vread = [&](int j) __attribute__((always_inline)) { return vfrag(vcur, j % DB, j / DB); };
    vf[0] = vread(0);
    vf[1] = vread(1);
    float mx = -INFINITY, rs = 0.f;
    const int thr = mask_thr(t + 1);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j % GAP == 0) {
        if (grpY)
          stage_copy<D, BN, NW>(kcur_w, rk, wave, j / GAP);
        else
          stage_copy<D, BN, NW>(vdst, rv, wave, j / GAP);
      }
      if (j + 2 < NB) vf[(j + 2) % 3] = vread(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int g = j / DB, db = j % DB;
      acc[db] = T::mfma(vf[j % 3], pf[g], acc[db]);
      if (g + 1 < NG) {
        const int gn = g + 1;
        constexpr int PPC = DB >= 4 ? 1 : 4 / DB;
#pragma unroll
        for (int c = 0; c < PPC; ++c) {
          const int w = db * PPC + c;
          if (w < 4) pf[gn].v[w] = T::pack2(s[gn / 2][8 * (gn % 2) + 2 * w], s[gn / 2][8 * (gn % 2) + 2 * w + 1]);
        }
      }
#pragma unroll
      for (int e = 0; e < NE / NB; ++e) {
        const int idx = j * (NE / NB) + e;
        rs += s[idx / 16][idx % 16];
        float x = sn_pp[idx / 16][idx % 16];
        if (MASK) {
          x = masked(x, idx / 16, idx % 16, thr);
          sn_pp[idx / 16][idx % 16] = x;
        }
        mx = fmaxf(mx, x);
      }
      asm volatile("" : "+v"(mx), "+v"(rs));
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = __builtin_fmaf(l_run, alpha, rs);
    update_ref(mx);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = sn_pp[kb];
  };

  // ---- last tile: P and P V only.
  auto drain = [&](auto parity_tag) __attribute__((always_inline)) {
    constexpr int P = decltype(parity_tag)::value;
    Frag pf[KB][2];
    softmax_p(s, pf);
    rescale();
    pv(P ? lds_v1 : lds_v0, pf);
  };

  using F = std::false_type;
  using Tr = std::true_type;
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  // Steps whose next tile needs no mask: t + 1 < n_plain.
  const int plain_steps = max(t0, min(n_plain - 1, last));
  if constexpr (NW == 8) {
    // Ping-pong of the two 4-wave groups sharing each SIMD: group Y (waves 4..7) runs half a
    // step behind group X (waves 0..3), so on every SIMD one wave is in its exponential-heavy
    // [A] half while the other is in its product-heavy [B] half. Every half-step ends with a
    // workgroup barrier. In half-step k every wave copies its share of one tile: K(t0 + k/2 + 2)
    // for even k, V(t0 + (k-1)/2 + 1) for odd k, into the slot the previous half-step freed;
    // the copies of half-step k must have landed by the end of half-step k+1.
    constexpr int CPWP = BN * D * 2 / 1024 / NW;  // copies per wave per tile
    const bool grpY = wave >= 4;
    auto end_slot = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | CPWP);  // vmcnt(CPWP): the previous half-step's copies landed
      ring_barrier();
    };
    // copy c of this wave's share of K(tk) into slot (tk - t0) & 1
    auto copy_k = [&](int tk, int c) __attribute__((always_inline)) {
      const int tt = min(tk, last);
      const TileSrc r = tile_src<D, BN>(Kh, tt * BN, NK, rsk, dh);
      if (((tk - t0) & 1) == 0) stage_copy<D, BN, NW>(lds_k0, r, wave, c);
      else stage_copy<D, BN, NW>(lds_k1, r, wave, c);
    };
    if (grpY) {
      // Y's idle first half-step: its share of K(t0 + 2)
#pragma unroll
      for (int c = 0; c < CPWP; ++c) copy_k(t0 + 2, c);
      end_slot();
    }
    int t = t0;
    auto pp_pair = [&](auto mask_tag, int tt) __attribute__((always_inline)) {
      half_a(mask_tag, Even(), tt, grpY);
      end_slot();
      half_b(mask_tag, Even(), tt, grpY);
      end_slot();
      half_a(mask_tag, Odd(), tt + 1, grpY);
      end_slot();
      half_b(mask_tag, Odd(), tt + 1, grpY);
      end_slot();
    };
    for (; t + 1 < plain_steps; t += 2) pp_pair(F(), t);
    for (; t < last; t += 2) {
      half_a(Tr(), Even(), t, grpY);
      end_slot();
      half_b(Tr(), Even(), t, grpY);
      end_slot();
      if (t + 1 < last) {
        half_a(Tr(), Odd(), t + 1, grpY);
        end_slot();
        half_b(Tr(), Odd(), t + 1, grpY);
        end_slot();
      }
    }
    // X pads one half-step with a full wait, so that every copy of V(last) (issued in X's and
    // Y's previous half-step) has landed; then both groups drain together.
    if (!grpY) {
      wait_async();
      ring_barrier();
    }
    if ((last - t0) & 1)
      drain(Odd());
    else
      drain(Even());
    wait_async();
    ring_barrier();
  } else if constexpr (RING == 2) {
  int t = t0;
  for (; t + 1 < plain_steps; t += 2) {
    step(F(), Even(), t);
    step(F(), Odd(), t + 1);
  }
  for (; t < last; t += 2) {
    step(Tr(), Even(), t);
    if (t + 1 < last) step(Tr(), Odd(), t + 1);
  }
  if ((last - t0) & 1)
    drain(Odd());
  else
    drain(Even());
  } else {
  int t = t0;
  for (; t + 2 < plain_steps; t += 3) {
    step(F(), S0(), t);
    step(F(), S1(), t + 1);
    step(F(), S2(), t + 2);
  }
  for (; t < last; t += 3) {
    step(Tr(), S0(), t);
    if (t + 1 < last) step(Tr(), S1(), t + 1);
    if (t + 2 < last) step(Tr(), S2(), t + 2);
  }
  // The last step's copies (clamped repeats of the last tiles, into free slots) land before
  // the workgroup moves on; V(last) itself landed before the last step's barrier. Its slot is
  // picked at run time: one drain body instead of three.
  wait_async();
  const int ph = (last - t0) % 3;
  const uint16_t* vlast = ph == 0 ? lds_v0 : (ph == 1 ? lds_v1 : lds_v2);
  Frag pf[KB][2];
  softmax_p(s, pf);
  rescale();
  pv(vlast, pf);
  }

  // ---- epilogue: one division per row, store O and LSE
  const float l_tot = MSUM ? lsum[0] : half_swap_sum(l_run);
  if (SPLIT) {
    if (qrow < N) {
      const size_t r = (size_t)sp * rows_all + sq_.stat + qrow;
      float* po = part + r * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g + 4 * h) =
              f32x4{acc[db][4 * g + 0], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
      if (h == 0) {
        part[(size_t)splits * rows_all * D + r] = l_tot > 0.f ? m_ref : -INFINITY;
        part[(size_t)splits * rows_all * (D + 1) + r] = l_tot;
      }
    }
    continue;
  }
  // a row that saw no key (l = 0) gets O = 0 and LSE = -inf
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = Oh + (size_t)qrow * rso;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv);
        w[1] = T::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
        // columns db*32 + 8g + 4h .. +3 exist iff db*32 + 8g < dh (dh is a multiple of 8)
        if (db * 32 + 8 * g < dh) *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * h) = w;
      }
    if (LSE != nullptr && h == 0) LSE[sq_.stat + qrow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
  }  // pass
}

// ------------------------------------------------------------------------------------------
// Merge of the split-KV partial states ("FlashAttentionを1から", section "その後の版と、推論での
// 事情"; the same algebra as the online softmax update). Per row, with m_s in log2 units:
//   M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,  O = (sum_s w_s acc_s) / L,
//   LSE = ln2 * (M + log2 L).
// An empty state (m_s = -inf, l_s = 0, acc_s = 0) gets weight 0. D/4 threads per row, 4
// elements each (16-byte loads of the fp32 partials); a block covers RPB consecutive rows of
// one statistics head (nrb blocks per head).
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part, uint16_t* __restrict__ O,
                                                    float* __restrict__ LSE, Geom geo, Strides so, long long rows,
                                                    int nrb, int splits) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  const int hh = blockIdx.x / nrb;
  const int r = (blockIdx.x - hh * nrb) * RPB + threadIdx.x / TPR;
  if (r >= stat_rows(geo)) return;
  const long long row = (long long)hh * stat_rows(geo) + r;
  const float* pm = part + (size_t)splits * rows * D;
  const float* pl = pm + (size_t)splits * rows;
  float M = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, pm[(size_t)sp * rows + row]);
  const float Mr = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const size_t r = (size_t)sp * rows + row;
    const float w = __builtin_amdgcn_exp2f(pm[r] - Mr);
    L = __builtin_fmaf(w, pl[r], L);
    const f32x4 o = *reinterpret_cast<const f32x4*>(part + r * D + sub * 4);
    a0 = __builtin_fmaf(w, o[0], a0);
    a1 = __builtin_fmaf(w, o[1], a1);
    a2 = __builtin_fmaf(w, o[2], a2);
    a3 = __builtin_fmaf(w, o[3], a3);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;  // a row that saw no key: O = 0, LSE = -inf
  u32x2 w2;
  w2[0] = T::pack2(a0 * inv, a1 * inv);
  w2[1] = T::pack2(a2 * inv, a3 * inv);
  if (sub * 4 < geo.dh) *reinterpret_cast<u32x2*>(O + stat_row_offset(geo, so, hh, r) + sub * 4) = w2;
  if (sub == 0 && LSE != nullptr) LSE[row] = L > 0.f ? (Mr + __log2f(L)) * kLn2 : -INFINITY;
}

template <typename T, int D>
static hipError_t launch_merge_t(const FwdArgs& a) {
  constexpr int RPB = 256 / (D / 4);
  const long long rows = (long long)stat_heads(a.g) * stat_rows(a.g);
  const int nrb = (stat_rows(a.g) + RPB - 1) / RPB;
  const long long grid = (long long)stat_heads(a.g) * nrb;
  if (grid == 0) return hipSuccess;
  return launch_kernel(&merge_kernel<T, D>, (unsigned)grid, 256, a.stream, a.part, (uint16_t*)a.o, a.lse, a.g, a.so,
                       rows, nrb, a.splits);
}

static hipError_t launch_merge(const FwdArgs& a) {
  if (a.bf16)
    return a.d <= 64 ? launch_merge_t<BF16, 64>(a) : a.d <= 128 ? launch_merge_t<BF16, 128>(a) : launch_merge_t<BF16, 256>(a);
  return a.d <= 64 ? launch_merge_t<FP16, 64>(a) : a.d <= 128 ? launch_merge_t<FP16, 128>(a) : launch_merge_t<FP16, 256>(a);
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  constexpr int NW = 4, BN = 64;
  if constexpr (D == 128) if (a.pingpong && a.splits == 0) {
    // the two-group ping-pong: 8 waves, 256 query rows per workgroup
    constexpr int NWP = 8, BMP = NWP * 32;
    const int nqt = (a.g.N + BMP - 1) / BMP;
    const int BHp = a.g.B * a.g.H;
    const bool pairp = CAUSAL && pair_causal_tiles((long long)((nqt + 1) / 2) * BHp * 2);
    const long long gridp = (long long)(pairp ? (nqt + 1) / 2 : nqt) * BHp;
    if (gridp == 0) return hipSuccess;
    return launch_kernel(&fwd_kernel<T, D, BN, NWP, CAUSAL, false>, (unsigned)gridp, NWP * 64, a.stream,
                         (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.g,
                         a.sq, a.sk, a.sv, a.so, nqt, pairp ? 1 : 0, a.c_log2, nullptr, 0LL, 0);
  }
  constexpr int BM = NW * 32;
  const int n_qtiles = (a.g.N + BM - 1) / BM;
  const int BH = a.g.B * a.g.H;
  if (a.splits > 0) {
    const long long grid = (long long)n_qtiles * a.splits * BH;
    const long long rows_all = (long long)stat_heads(a.g) * stat_rows(a.g);
    if (grid > 0) {
      const hipError_t e = launch_kernel(&fwd_kernel<T, D, BN, NW, CAUSAL, true>, (unsigned)grid, NW * 64, a.stream,
                                         (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                                         (uint16_t*)a.o, a.lse, a.g, a.sq, a.sk, a.sv, a.so, n_qtiles, 0, a.c_log2,
                                         a.part, rows_all, a.splits);
      if (e != hipSuccess) return e;
    }
    return launch_merge(a);
  }
  const bool pair = CAUSAL && pair_causal_tiles((long long)((n_qtiles + 1) / 2) * BH);
  const long long grid = (long long)(pair ? (n_qtiles + 1) / 2 : n_qtiles) * BH;
  if (grid == 0) return hipSuccess;
  return launch_kernel(&fwd_kernel<T, D, BN, NW, CAUSAL, false>, (unsigned)grid, NW * 64, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.g,
                       a.sq, a.sk, a.sv, a.so, n_qtiles, pair ? 1 : 0, a.c_log2, nullptr, 0LL, 0);
}

template <typename T>
static hipError_t launch_fwd_dt(const FwdArgs& a) {
  if (a.d <= 64) return a.causal ? launch_fwd_t<T, 64, true>(a) : launch_fwd_t<T, 64, false>(a);
  if (a.d <= 128) return a.causal ? launch_fwd_t<T, 128, true>(a) : launch_fwd_t<T, 128, false>(a);
  return a.causal ? launch_fwd_t<T, 256, true>(a) : launch_fwd_t<T, 256, false>(a);
}

hipError_t launch_forward(const FwdArgs& a) {
  return a.bf16 ? launch_fwd_dt<BF16>(a) : launch_fwd_dt<FP16>(a);
}

}  // namespace fa
