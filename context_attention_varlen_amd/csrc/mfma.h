// Device building blocks of the bf16 attention kernels on gfx950:
// v_mfma_f32_32x32x16_bf16 operand layouts, swizzled row-major LDS tiles
// filled by direct global->LDS loads, and transposed operand reads.
#pragma once

#include "common.h"

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// MFMA 32x32x16 bf16 layouts (lane l, half hh = l / 32, col = l % 32):
//   A[m][k]: lane holds row m = col, 8 k-values (slot e of half hh)
//   B[k][n]: lane holds column n = col, 8 k-values (slot e of half hh)
//   C[m][n]: lane holds column n = col, rows 8*(i/4) + 4*hh + i%4, i = 0..15
// A and B assign (hh, e) to the same k, so any consistent k-order works.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row-major bf16 tile of D columns in LDS, 16-byte chunks XOR-swizzled by
//   f(row) = ((row & 3) << (log2(D/8) - 2)) | ((row >> 2) & (D/32 - 1)).
// 16 (D=128) or 8 (D=64) consecutive rows read at one logical chunk land in
// distinct chunks (row-wise 128-bit reads), and 4 consecutive rows x 4
// (or 2) adjacent chunks land in distinct chunks (transposed reads).
template <int D>
__device__ __forceinline__ int swz(int row) {
  constexpr int KCH = D / 8;
  constexpr int SH = KCH == 16 ? 2 : 1;
  return ((row & 3) << SH) | ((row >> 2) & (KCH / 4 - 1));
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + ((chunk ^ swz<D>(row)) << 3);
}

// Direct global -> LDS copy of rows [t0, t0 + R) of a segment (rows past the
// segment end repeat its last row: finite data that the mask discards) into
// an R x D swizzled tile.  Every wave issues NINST/NW 1-KiB loads; lane p of
// a load fetches the global chunk that belongs at LDS chunk p.
template <int D, int R, int NW>
__device__ __forceinline__ void load_tile(uint16_t* lds, const uint16_t* gbase, int64_t row_stride, int srow,
                                          int t0, int n, int wave, int lane) {
  constexpr int KCH = D / 8;
  constexpr int NINST = R * KCH / 64;
  static_assert(NINST % NW == 0, "tile loads split evenly over waves");
#pragma unroll
  for (int i = 0; i < NINST / NW; ++i) {
    const int q = i * NW + wave;
    const int p = q * 64 + lane;
    const int row = p / KCH;
    const int c = (p % KCH) ^ swz<D>(row);
    const int r = min(t0 + row, n - 1);
    const uint16_t* src = gbase + (int64_t)(srow + r) * row_stride + c * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(lds + q * 512), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte row read: A (or B) operand slot for row `row`, logical chunk `chunk`.
template <int D>
__device__ __forceinline__ bf16x8 read_row8(const uint16_t* tile, int row, int chunk) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)(tile + tile_off<D>(row, chunk)));
}

// Transposed operand: the 32 x 16 operand whose MFMA row index runs along
// tile columns [c0, c0 + 32) and whose k index runs along tile rows
// [r0, r0 + 16).  With ds_read_b64_tr_b16, lane j of each 16-lane group
// points at tile[rb + j/4][cb + 4*(j%4)] and receives tile[rb + e][cb + j]
// for e = 0..3.  Slot e = 4t + e' of half hh holds tile row
// r0 + 8t + 4hh + e', matching the C layout rows of a 32-row block split
// into two 16-row k-steps.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const uint16_t* tile, int r0, int c0, int lane) {
  const int j = lane & 15, mh = (lane >> 4) & 1, hh = lane >> 5;
  const int col = c0 + 16 * mh + 4 * (j & 3);
  s16x4 v[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = r0 + 8 * t + 4 * hh + (j >> 2);
    const int off = row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
    v[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + off));
  }
  u32x4 r;
  r[0] = __builtin_bit_cast(u32x2, v[0])[0];
  r[1] = __builtin_bit_cast(u32x2, v[0])[1];
  r[2] = __builtin_bit_cast(u32x2, v[1])[0];
  r[3] = __builtin_bit_cast(u32x2, v[1])[1];
  return __builtin_bit_cast(bf16x8, r);
}

// B operand from a C-layout accumulator (16 rows per half) for k-step ps of
// a 32-row block: slot e takes C register 8*(ps % 2) + e, i.e. rows
// 16*(ps%2) + 8*(e/4) + 4*hh + e%4, the same rows read_tr puts in slot e.
__device__ __forceinline__ bf16x8 pack_b(const f32x16& c, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[8 * half + e];
  return r;
}

// blockIdx -> (item rank, kv-head, index inside the GQA group).  The G
// workgroups of one (item, kv-head) unit occupy consecutive dispatch slots
// of one XCD (slots go round-robin over the 8 XCDs), and units are dealt to
// XCDs in item order, so each XCD works on a fixed set of kv-heads when Hkv
// divides 8 or 8 divides Hkv: their K/V stay in that XCD's L2.
__device__ __forceinline__ void map_block(int bid, int grp, int hkv, int& item_rank, int& head, int& kvh) {
  const int x = bid & 7;
  const int k = bid >> 3;
  const int u = k / grp, j = k - u * grp;
  const int U = u * 8 + x;
  item_rank = U / hkv;
  kvh = U - item_rank * hkv;
  head = kvh * grp + j;
}

inline unsigned unit_grid(int64_t max_items, int hkv, int grp) {
  const int64_t units = max_items * hkv;
  return (unsigned)(((units + 7) / 8) * 8 * grp);
}

}  // namespace cpattn
