// Device-side building blocks shared by the gfx950 attention kernels:
// element types, the MFMA tiles, LDS fragment loads and fp32 -> 16-bit rounding.
//
// MFMA tile used everywhere: v_mfma_f32_32x32x16_{bf16,f16}, D(32x32,fp32) += A(32x16) B(16x32).
// Lane layout (wave64, lane l, h = l/32, l32 = l%32), verified on gfx950:
//   A operand : lane l holds A[m = l32][k = 8h + j], j = 0..7     (8 x 16-bit, one VGPR quad)
//   B operand : lane l holds B[k = 8h + j][n = l32], j = 0..7
//   D         : lane l, register i (0..15) holds D[m = 8(i/4) + 4h + (i%4)][n = l32]
// So each lane owns one output column n and 16 rows of it. Register group t (i = 8t..8t+7)
// of a D tile covers rows 16t + sigma_h(j), sigma_h(j) = 8(j/4) + 4h + (j%4); converted to
// 16-bit, it is exactly the B operand of a k=16 step whose k index runs over those same
// rows in the order sigma_h. Any A operand paired with it must use the same k order,
// which the transposing LDS read below provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.hpp"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

// 8 packed 16-bit elements = one MFMA operand per lane.
struct Frag {
  u32x4 v;
};

struct BF16 {
  typedef __bf16 elem;
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma(const Frag& a, const Frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
  // Two fp32 -> packed pair of bf16, round to nearest even (one v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  }
};

struct FP16 {
  typedef _Float16 elem;
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma(const Frag& a, const Frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.v),
                                                  __builtin_bit_cast(f16x8, b.v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
};

// ---------------------------------------------------------------------------------------
// Lane coordinates.
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------------------
// Register group t (8 fp32 values, i = 8t..8t+7) of a D tile -> 16-bit operand fragment.
template <typename T>
__device__ __forceinline__ Frag pack_group(const f32x16& d, int t) {
  Frag f;
  f.v[0] = T::pack2(d[8 * t + 0], d[8 * t + 1]);
  f.v[1] = T::pack2(d[8 * t + 2], d[8 * t + 3]);
  f.v[2] = T::pack2(d[8 * t + 4], d[8 * t + 5]);
  f.v[3] = T::pack2(d[8 * t + 6], d[8 * t + 7]);
  return f;
}

// ---------------------------------------------------------------------------------------
// LDS tiles hold 16-bit elements row-major with a row stride of `stride` elements.

// Operand with k contiguous in memory: lane gets Mem[row0 + l32][k0 + 8h .. k0 + 8h + 7].
// Serves as an A operand (rows = m) or a B operand (rows = n). One 16-byte LDS read.
__device__ __forceinline__ Frag lds_frag_rows(const uint16_t* base, int stride, int row0, int k0) {
  const int l = lane_id();
  const uint16_t* p = base + (row0 + (l & 31)) * stride + k0 + ((l >> 5) << 3);
  Frag f;
  f.v = *reinterpret_cast<const u32x4*>(p);
  return f;
}

// Operand whose k index runs down the rows of a row-major tile (the transpose of the tile):
// lane gets Mem[krow0 + sigma_h(j)][m0 + l32] for j = 0..7, i.e. A[m][k] = Mem[k][m] with
// k in the sigma order that matches pack_group(). Two ds_read_b64_tr_b16: within each group
// of 16 lanes, source lane s addresses row (s/4) of a 4-row block at column 4(s%4); lane r of
// the group receives column r of those 4 rows.
__device__ __forceinline__ Frag lds_frag_cols(const uint16_t* base, int stride, int krow0, int m0) {
  const int l = lane_id();
  const int h = l >> 5;
  const int col = m0 + (((l >> 4) & 1) << 4) + ((l & 3) << 2);
  const int rsub = (l & 15) >> 2;
  const uint16_t* p0 = base + (krow0 + 4 * h + rsub) * stride + col;
  const uint16_t* p1 = p0 + 8 * stride;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p1));
  Frag f;
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 ub = __builtin_bit_cast(u32x2, b);
  f.v[0] = ua[0];
  f.v[1] = ua[1];
  f.v[2] = ub[0];
  f.v[3] = ub[1];
  return f;
}

// ---------------------------------------------------------------------------------------
// Swizzled tiles: rows of D 16-bit elements (D/8 chunks of 16 bytes), no padding, with
// chunk c of row r stored at chunk c ^ swz(r). The row permutation makes both access
// patterns the kernels use on the same tile free of LDS bank conflicts (64 banks x 4 B):
//   row reads  - 16 lanes read one 16-byte chunk from 16 consecutive rows;
//   transposing reads - 32 lanes read 8 bytes each from 4 consecutive rows x 4 chunks;
// and keeps the 16-byte staging writes (one row per 16 lanes) conflict-free too.
//   D = 128 (16 chunks): swz(r) = bits (r1 r0 r3 r2) of r, i.e. ((r & 3) << 2) | ((r >> 2) & 3)
//   D = 64  (8 chunks, two rows per bank line): swz(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128 || D == 256, "swizzle defined for tile widths 64, 128 and 256");
  // 256 wide (32 chunks, 512-byte rows): the 128-wide permutation on the low 4 chunk bits;
  // rows are a whole number of bank lines apart in both, so the bank pattern of every read
  // is the same as at 128
  return D >= 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Element offset of (row, col) in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row)) << 3) | (col & 7));
}

// lds_frag_rows() on a swizzled tile.
template <int D>
__device__ __forceinline__ Frag swz_frag_rows(const uint16_t* base, int row0, int k0) {
  const int l = lane_id();
  Frag f;
  f.v = *reinterpret_cast<const u32x4*>(base + swz_off<D>(row0 + (l & 31), k0 + ((l >> 5) << 3)));
  return f;
}

// lds_frag_cols() on a swizzled tile (each 8-byte transposing read stays inside a chunk).
template <int D>
__device__ __forceinline__ Frag swz_frag_cols(const uint16_t* base, int krow0, int m0) {
  const int l = lane_id();
  const int h = l >> 5;
  const int col = m0 + (((l >> 4) & 1) << 4) + ((l & 3) << 2);
  const int row = krow0 + 4 * h + ((l & 15) >> 2);
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(base + swz_off<D>(row, col)));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(base + swz_off<D>(row + 8, col)));
  Frag f;
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 ub = __builtin_bit_cast(u32x2, b);
  f.v[0] = ua[0];
  f.v[1] = ua[1];
  f.v[2] = ub[0];
  f.v[3] = ub[1];
  return f;
}

// Fragment reads at per-lane byte offsets that already carry every XOR term of the swizzle
// (precomputed from swz_rows_base / swz_cols_base below); what is left of the address is a
// compile-time add that lands in the instruction's offset field, so a read costs no VALU.
__device__ __forceinline__ Frag lds_read_rows(const uint16_t* tile, int ofs) {
  Frag f;
  f.v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(tile) + ofs);
  return f;
}
// Transposing read pair: the first 8-byte read at ofs0 (rows krow0 + 4h + (l&15)/4), the second
// at ofs1 (8 rows further down).
__device__ __forceinline__ Frag lds_read_cols(const uint16_t* tile, int ofs0, int ofs1) {
  const char* b = reinterpret_cast<const char*>(tile);
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + ofs0));
  i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + ofs1));
  Frag f;
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 uc = __builtin_bit_cast(u32x2, c);
  f.v[0] = ua[0];
  f.v[1] = ua[1];
  f.v[2] = uc[0];
  f.v[3] = uc[1];
  return f;
}

// ---------------------------------------------------------------------------------------
// Workgroup -> (head, tile) mapping that keeps a head's tiles on one XCD.
// The dispatcher deals workgroups round-robin over the 8 XCDs (blockIdx.x % 8), and each
// XCD has its own L2. Renumbering so that the workgroups one XCD receives in a row are the
// consecutive tiles of the same head lets the tiles of a head that run together share its
// K/V (or Q/dO) reads in that XCD's L2 instead of each XCD cycling through every head.
// `total` = number of workgroups; returns the logical index in [0, total), head-major.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_local_index(int bid, int total) {
  const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const int per = total / kNumXcd, rem = total % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Logical head index (the rank of a head in the order work items are dealt out) to b*H + h,
// with the batch index running fastest. Each XCD takes a contiguous range of logical heads,
// so in a packed batch every XCD then holds an equal share of every sequence. With b slowest,
// an XCD would hold whole sequences, and the one that drew the longest would set the time.
// A bijection on [0, B*H): every head is still visited exactly once.
__device__ __forceinline__ int head_of_item(int lbh, int B, int H) { return (lbh % B) * H + lbh / B; }

// Per-lane base offsets into a swizzled tile, from which every fragment address follows by
// an XOR with a compile-time constant (the swizzle is linear over XOR) plus a constant add:
//  * row reads at (row0 + l32, chunk 2ks + h): element offset = rows_base(row0) ^ (ks << 4);
//  * transposing reads at rows krow0 + 4h + (l&15)/4 (+8), columns m0 + 16((l>>4)&1) + 4(l&3),
//    krow0 % 16 == 0, m0 % 32 == 0: first read cols_base + krow0*D ^ ((m0/32) << 5); the
//    second (8 rows down) flips swizzle bit 1 (element bit 4) and adds 8 rows.
// Valid because swz(r + 16) = swz(r), swz(r + 8) = swz(r) ^ 2, and chunk bits added by ks and
// m0 never overlap the bits h, (l>>4)&1 and (l&3)>>1 occupy.
template <int D>
__device__ __forceinline__ int swz_rows_base(int row0) {
  const int l = lane_id();
  return swz_off<D>(row0 + (l & 31), (l >> 5) << 3);
}
template <int D>
__device__ __forceinline__ int swz_cols_base() {
  const int l = lane_id();
  return swz_off<D>(4 * (l >> 5) + ((l & 15) >> 2), (((l >> 4) & 1) << 4) + ((l & 3) << 2));
}
template <int D>
__device__ __forceinline__ Frag swz_rows_frag(const uint16_t* tile, int base, int ks) {
  Frag f;
  f.v = *reinterpret_cast<const u32x4*>(tile + (base ^ (ks << 4)));
  return f;
}
template <int D>
__device__ __forceinline__ Frag swz_cols_frag(const uint16_t* tile, int base, int krow0, int m0) {
  const int o0 = (base ^ ((m0 >> 5) << 5)) + krow0 * D;
  const int o1 = (o0 ^ 16) + 8 * D;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tile + o0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tile + o1));
  Frag f;
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 ub = __builtin_bit_cast(u32x2, b);
  f.v[0] = ua[0];
  f.v[1] = ua[1];
  f.v[2] = ub[0];
  f.v[3] = ub[1];
  return f;
}

// ---------------------------------------------------------------------------------------
// Asynchronous global -> LDS staging with buffer_load_dwordx4 ... lds (MUBUF): one wave
// instruction copies 64 x 16 bytes into LDS bytes [M0, M0 + 1024), lane i landing at
// M0 + 16 i, with no VGPR round trip; completion is tracked by vmcnt, and wait_async() plus a
// barrier publishes the data. (The FLAT-encoded global_load_lds would do the same copy, but
// while a FLAT instruction that may touch LDS is in flight the compiler's wait insertion
// cannot tell it from an LDS read and flushes lgkmcnt to zero before every LDS operand use,
// which serialises read-ahead fragment loads.)
//
// A descriptor covers just the rows that exist: reads at or past its size return zero (the
// hardware range check), finite data that the kernels mask, and no load leaves the tensor.
// Word 3 (0x00020000) is the gfx9 setting for untyped 32-bit access. Base and size are
// wave-uniform by contract; readfirstlane pins them to SGPRs (a descriptor the compiler sees
// in VGPRs turns each copy into a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Source of a ROWS-row tile: one descriptor over rows [grow0, grow0 + ROWS) of a head whose
// rows are rs elements apart and dh <= D elements wide, ending with the last existing row's
// dh elements (empty if none exists), so every row at or past n_rows reads as zero.
// Wave-uniform.
struct TileSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  int rs, dh;
};
template <int D, int ROWS>
__device__ __forceinline__ TileSrc tile_src(const uint16_t* head, int grow0, int n_rows, int rs, int dh) {
  TileSrc t;
  const int avail = __builtin_amdgcn_readfirstlane(max(0, min(n_rows - grow0, ROWS)));
  t.rsrc = make_rsrc(head + (size_t)grow0 * rs, avail > 0 ? ((avail - 1) * rs + dh) * 2 : 0);
  t.rs = rs;
  t.dh = dh;
  return t;
}
// A source offset no descriptor reaches (sizes stay below 2^31): the range check returns
// zero for it without touching memory.
constexpr int kOffOutOfRange = (int)0x80000000u;
// Copy k (0 <= k < ROWS*D*2/1024/NW) of wave `wave`'s share of a ROWS-row tile of D 16-bit
// elements: 1 KB, i.e. RPI = 1024/(2D) whole rows starting at row ins*RPI, ins = wave + k*NW,
// landing swizzled at tile[ins * 512 ...]. The per-lane part of the source offset (row within
// the copy, swizzled chunk) is the same for every copy of a wave, because successive copies
// move by NW*RPI rows, a whole number of swizzle periods; the copy's row shift is added per
// issue (the hardware range check sees the whole offset). The compiler hoists each copy's
// sum out of the loop (one register per copy); with SHARED_OFS the lane part is made opaque
// instead, so one register serves every copy at the price of an add (and a move) per issue,
// for kernels without registers to spare. Every wave issues the same, compile-time number of
// copies, so the compiler's vmcnt bookkeeping is exact.
template <int D, int ROWS, int NW, bool SHARED_OFS = false>
__device__ __forceinline__ void stage_copy(uint16_t* tile, const TileSrc& src, int wave, int k) {
  constexpr int ROW_BYTES = D * 2;
  constexpr int RPI = 1024 / ROW_BYTES;  // rows per copy
  constexpr int LPR = ROW_BYTES / 16;    // lanes per row
  static_assert((ROWS * ROW_BYTES / 1024) % NW == 0, "tile copies must split evenly over the waves");
  constexpr bool PERIODIC = (NW * RPI) % 16 == 0;  // a wave's copies sit whole swizzle periods apart
  static_assert(PERIODIC || !SHARED_OFS, "a shared lane offset needs copies whole swizzle periods apart");
  const int ins = wave + k * NW;
  const int l = lane_id();
  const int lrow = l / LPR;
  // = swz(ins*RPI + lrow) when PERIODIC (period 16)
  const int chunk = (l % LPR) ^ swz<D>((PERIODIC ? wave : ins) * RPI + lrow);
  // columns past the operand's head dim read as zero
  int lane_ofs = chunk * 8 < src.dh ? lrow * src.rs * 2 + (chunk << 4) : kOffOutOfRange;
  if (SHARED_OFS) asm volatile("" : "+v"(lane_ofs));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rsrc, (FA_LDS void*)(tile + ins * 512), 16,
                                           lane_ofs + ins * (RPI * 2) * src.rs, 0, 0, 0);
}
// All of wave `wave`'s copies of the tile at rows [grow0, grow0 + ROWS).
template <int D, int ROWS, int NW, bool SHARED_OFS = false>
__device__ __forceinline__ void stage_rows_swz_buf(uint16_t* tile, const uint16_t* head, int grow0, int n_rows, int rs,
                                                   int dh, int wave) {
  const TileSrc src = tile_src<D, ROWS>(head, grow0, n_rows, rs, dh);
#pragma unroll
  for (int k = 0; k < ROWS * D * 2 / 1024 / NW; ++k) stage_copy<D, ROWS, NW, SHARED_OFS>(tile, src, wave, k);
}

// Per-row statistics of 32 rows from two arrays: dst[0..31] = a[r0 ..], dst[64..95] =
// b[r0 ..] (dst holds 128 floats; [32..63] and [96..127] receive copies of the same values).
// Two full-wave copies with one descriptor each: lane-divergent copies from two descriptors
// get merged by the compiler into one copy with a per-lane descriptor.
constexpr int kStatB = 64;  // offset of the second array's values in a statistics slot
// dst is an LDS pointer already (cast from the __shared__ array itself), so no generic-to-LDS
// conversion with its null test is left for the compiler to place.
__device__ __forceinline__ void stage_stats_buf(FA_LDS float* dst, const float* a, const float* b, int r0, int n_rows) {
  const int voff = (lane_id() & 31) * 4;
  const int avail = max(0, min(n_rows - r0, 32));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a + r0, avail * 4), (FA_LDS void*)dst, 4, voff, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(b + r0, avail * 4), (FA_LDS void*)(dst + kStatB), 4, voff, 0, 0,
                                           0);
}

// vmcnt(0) through the builtin rather than inline asm, so the compiler's wait-insertion pass
// knows every copy has completed (immediate: vmcnt 0, expcnt 7, lgkmcnt 15).
__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for loops that keep asynchronous LDS copies in flight across it.
// __syncthreads() carries a workgroup release fence, which makes the compiler wait for every
// outstanding copy (vmcnt(0)) first; here the caller waits for exactly the copies the next
// iteration reads, and only this wave's own LDS reads must have completed (lgkmcnt(0)) so no
// other wave's copy can overwrite data still being read.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Global 16-byte load of 8 elements (zero when !valid).
__device__ __forceinline__ u32x4 gload16(const uint16_t* p, bool valid) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return valid ? *reinterpret_cast<const u32x4*>(p) : z;
}

__device__ __forceinline__ float wave_xor32_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float wave_xor32_sum(float x) {
  return x + __shfl_xor(x, 32, 64);
}

// The same two reductions through v_permlane32_swap (a VALU op: no LDS round trip and no
// lgkmcnt, so it does not wait behind outstanding LDS reads). Swapping x with itself leaves
// x_l and x_(l^32) in the two results on every lane, in some order; max and sum do not care.
__device__ __forceinline__ float half_swap_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier (the AMDGPU backend's
// SchedGroupMask): a sequence of group barriers tells the scheduler how to interleave
// matrix-core, vector-ALU and LDS instructions inside one basic block.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedTrans = 0x400;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The sequence a workgroup works on: head bh = b*H + h of the grid, its query and key
// lengths n and nk, the packed rows its query and key row 0 are (0 for fixed lengths) and the
// index of its query row 0 in LSE / delta. Values read from cu / cuk are clamped
// (0 <= row0 <= row0 + n <= T, n <= N; likewise for the keys) and made wave-uniform.
struct Seq {
  int b, h, n, nk;
  long long row0, row0k, stat;
};
__device__ __forceinline__ Seq seq_of(const Geom& g, int bh) {
  Seq s;
  s.b = __builtin_amdgcn_readfirstlane(bh / g.H);
  s.h = __builtin_amdgcn_readfirstlane(bh - s.b * g.H);
  if (g.cu != nullptr) {
    const int c0 = min(max(__builtin_amdgcn_readfirstlane(g.cu[s.b]), 0), g.T);
    const int c1 = min(max(__builtin_amdgcn_readfirstlane(g.cu[s.b + 1]), c0), g.T);
    s.n = min(c1 - c0, g.N);
    s.row0 = c0;
    s.stat = (long long)s.h * g.T + c0;
    const int k0 = min(max(__builtin_amdgcn_readfirstlane(g.cuk[s.b]), 0), g.Tk);
    const int k1 = min(max(__builtin_amdgcn_readfirstlane(g.cuk[s.b + 1]), k0), g.Tk);
    s.nk = min(k1 - k0, g.Nk);
    s.row0k = k0;
  } else {
    s.n = g.N;
    s.nk = g.Nk;
    s.row0 = 0;
    s.row0k = 0;
    s.stat = (long long)bh * g.N;
  }
  return s;
}
// Row 0 of query-side operand `base` (strides st) for sequence s (with variable lengths the
// caller passes a zero batch stride: the packed row row0 already selects the sequence).
template <typename P>
__device__ __forceinline__ P* seq_base(P* base, const Strides& st, const Seq& s) {
  return base + ((long long)s.b * st.b + (long long)s.h * st.h + s.row0 * st.r);
}
// Row 0 of key-side operand `base` (K, V, dK, dV) for sequence s.
template <typename P>
__device__ __forceinline__ P* seq_base_k(P* base, const Strides& st, const Seq& s) {
  return base + ((long long)s.b * st.b + (long long)s.h * st.h + s.row0k * st.r);
}

// Statistics rows (LSE, delta, split-KV partial states) form (HH, Rh): HH = B*H heads of N
// rows each (fixed lengths) or H heads of T packed rows (variable lengths); see Geom.
__host__ __device__ __forceinline__ int stat_heads(const Geom& g) { return g.cu != nullptr ? g.H : g.B * g.H; }
__host__ __device__ __forceinline__ int stat_rows(const Geom& g) { return g.cu != nullptr ? g.T : g.N; }
// Element offset of statistics row (hh, r) in an operand with strides st.
__device__ __forceinline__ long long stat_row_offset(const Geom& g, const Strides& st, int hh, int r) {
  if (g.cu != nullptr) return (long long)hh * st.h + (long long)r * st.r;
  const int b = hh / g.H;
  return (long long)b * st.b + (long long)(hh - b * g.H) * st.h + (long long)r * st.r;
}

}  // namespace fa
