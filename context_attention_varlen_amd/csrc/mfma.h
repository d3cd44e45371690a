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

// bf16 tile of D columns in LDS, stored in 1 KiB blocks of RG = 512/D rows.
// Inside a block, 64-byte pieces (4 chunks of 16 bytes) of the RG rows are
// interleaved: piece cg = chunk/4 of row r sits at cg*RG*64 + (r%RG)*64
// bytes, and its 4 chunks are XOR-permuted by s(r) = (r/4) % 4:
//   offset(r, c) = (r/RG)*1024 + (c/4)*RG*64 + (r%RG)*64 + ((c%4) ^ s(r))*16.
// Modulo 256 bytes this is (r%4)*64 + ((c%4) ^ s(r))*16, so 16 consecutive
// rows read at one chunk (row-wise 128-bit reads) and 4 consecutive rows x 4
// adjacent chunks (transposed reads) both touch 16 distinct 16-byte bank
// slots. The chunk index enters only through c/4 (a constant for a given
// k-step) and c%4, so a lane needs two base addresses per tile and every
// k-step is an immediate offset from one of them. One direct-load
// instruction (64 lanes x 16 bytes) fills exactly one block.
//
// Element offset of chunk 4*cg + cl of row rc + rl, split so that the
// compiler sees which parts are constant: rc (constant or wave-uniform) is
// a multiple of 16, or a multiple of 8 with rl < 8; rl >= 0 is the
// lane-dependent row part, cg the constant chunk group and 0 <= cl < 4 the
// lane-dependent chunk part. Under those conditions (rc + rl)/4 % 4 equals
// (rc/4 % 4) ^ (rl/4 % 4).
template <int D>
__device__ __forceinline__ int tile_off_split(int rc, int rl, int cg, int cl) {
  constexpr int LRG = D == 128 ? 2 : 3;  // log2 of RG = 512 / D
  const unsigned urc = (unsigned)rc, url = (unsigned)rl, ucl = (unsigned)cl;
  const unsigned s = ((urc >> 2) & 3u) ^ ((url >> 2) & 3u);
  return (int)(((urc >> LRG) << 9) + ((url >> LRG) << 9) + ((url & ((1u << LRG) - 1)) << 5) +
               (unsigned)cg * (32u << LRG) + ((ucl ^ s) << 3));
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return tile_off_split<D>(0, row, chunk >> 2, chunk & 3);
}

// Buffer resource over `bytes` bytes from `base`: raw buffer loads at byte
// offsets past the end return zeros without touching memory (the hardware
// range check), which is how ragged tile tails are filled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct global -> LDS loads of an R x D bf16 tile into the LDS tile layout.
// Each wave issues PER loads of 1 KiB; lane p of load q fetches the global
// 16-byte chunk that belongs at LDS chunk q*64 + p.  Lane byte offsets and
// the wave-uniform LDS offsets are computed once; per tile only the scalar
// buffer base and the number of valid rows change (rows past it read as 0).
template <int D, int R, int NW>
struct TileLoader {
  static constexpr int KCH = D / 8;
  static constexpr int NINST = R * KCH / 64;
  static constexpr int PER = NINST / NW;
  static_assert(NINST % NW == 0, "tile loads split evenly over waves");
  static_assert(R % (512 / D) == 0, "whole 1 KiB blocks");
  int voff[PER];
  int ldso[PER];

  __device__ __forceinline__ void init(int64_t row_stride_bytes, int wave_u, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      // load q fills LDS block q: lane p lands at 16*p bytes into it
      constexpr int RG = 512 / D;
      const int q = i * NW + wave_u;
      const int row = q * RG + (lane >> 2) % RG;
      const int c = ((lane >> 2) / RG) * 4 + ((lane & 3) ^ ((row >> 2) & 3));
      voff[i] = (int)(row * row_stride_bytes) + c * 16;
      ldso[i] = q * 512;
    }
  }

  // rows [0, nvalid) of the tile start at `tile_base` (bytes), consecutive
  // rows `row_stride_bytes` apart
  __device__ __forceinline__ void issue(uint16_t* lds, const void* tile_base, int nvalid,
                                        int64_t row_stride_bytes) const {
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(tile_base, (unsigned)(nvalid * row_stride_bytes));
#pragma unroll
    for (int i = 0; i < PER; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + ldso[i]), 16,
                                               voff[i], 0, 0, 0);
  }
};

// Max of a value over the two 32-lane halves of the wave (the C-layout rows
// of one accumulator column live in lanes l and l^32).
// (v_max_f32 written out: fmaxf would first canonicalize both inputs, two
// more instructions, since the compiler cannot tell they are not NaNs)
__device__ __forceinline__ float max_halves(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(__uint_as_float(pr[0])), "v"(__uint_as_float(pr[1])));
  return r;
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Three-input max (v_max3_f32); the compiler forms few of these on its own.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// wait until at most `tiles` tile loads of PER instructions each are
// outstanding (0..3), issue order being the order they are needed in
template <int PER>
__device__ __forceinline__ void wait_vmcnt_tiles(int tiles) {
  if (tiles >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
  else if (tiles == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
  else if (tiles == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// 16-byte row read: the A (or B) operand slot of k-step ks for tile row
// rc + rl (rc a multiple of 16), i.e. chunk 2*ks + hh of that row.
typedef __attribute__((address_space(3))) const uint16_t lds_u16;

// LDS pointer of a tile: offsets added to it stay 32-bit, so constant parts
// fold into the instructions' immediate offsets
__device__ __forceinline__ lds_u16* lds_ptr(const uint16_t* tile) { return (lds_u16*)tile; }

template <int D>
__device__ __forceinline__ bf16x8 read_row8(const uint16_t* tile, int rc, int rl, int ks, int hh) {
  lds_u16* p = lds_ptr(tile) + tile_off_split<D>(rc, rl, ks >> 1, 2 * (ks & 1) + hh);
  return __builtin_bit_cast(bf16x8, *(__attribute__((address_space(3))) const u32x4*)p);
}

// tile_off_split as a constant part plus a lane part:
//   tile_off_split(rc, rl, cg, cl) == tile_off_const(rc, cg) + tile_off_lane(rl, cl ^ ((rc >> 2) & 3))
template <int D>
__device__ __forceinline__ int tile_off_const(int rc, int cg) {
  constexpr int LRG = D == 128 ? 2 : 3;
  return (int)((((unsigned)rc >> LRG) << 9) + (unsigned)cg * (32u << LRG));
}
template <int D>
__device__ __forceinline__ int tile_off_lane(int rl, int cl) { return tile_off_split<D>(0, rl, 0, cl); }

// A lane offset the optimizer cannot take apart.  Reads built as
// tile + opaque lane offset + constant keep every constant in the
// instruction's immediate offset and stay a short address chain from their
// LDS variable, so the compiler can tell a read of one LDS variable from
// direct loads still filling another and waits for the loads only where
// the buffers are the same.
__device__ __forceinline__ int opaque_lane(int x) {
  asm("" : "+v"(x));
  return x;
}

// read_row8 of k-step ks at tile row rc + (the lane's row), with lane_off
// = tile_off_lane(row, (2 * (ks & 1)) ^ hh) (rc a multiple of 16)
template <int D>
__device__ __forceinline__ bf16x8 read_row8_at(const uint16_t* tile, int lane_off, int rc, int ks) {
  lds_u16* p = lds_ptr(tile) + lane_off + tile_off_const<D>(rc, ks >> 1);
  return __builtin_bit_cast(bf16x8, *(__attribute__((address_space(3))) const u32x4*)p);
}

// read_tr with the lane parts precomputed: lane_off[t] =
// tile_off_lane(4hh + j/4, (2mh + (j%4)/2) ^ 2t) + 4(j%2) (r0 a multiple of 16)
template <int D>
__device__ __forceinline__ bf16x8 read_tr_at(const uint16_t* tile, const int (&lane_off)[2], int r0, int c0) {
  s16x4 v[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
    v[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(lds_ptr(tile) + lane_off[t] + tile_off_const<D>(r0 + 8 * t, c0 >> 5)));
  u32x4 r;
  r[0] = __builtin_bit_cast(u32x2, v[0])[0];
  r[1] = __builtin_bit_cast(u32x2, v[0])[1];
  r[2] = __builtin_bit_cast(u32x2, v[1])[0];
  r[3] = __builtin_bit_cast(u32x2, v[1])[1];
  return __builtin_bit_cast(bf16x8, r);
}

// The two lane offsets read_tr_at needs for this lane
template <int D>
__device__ __forceinline__ void tr_lane_offsets(int lane, int (&lane_off)[2]) {
  const int j = lane & 15, mh = (lane >> 4) & 1, hh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t)
    lane_off[t] = opaque_lane(tile_off_lane<D>(4 * hh + (j >> 2), (2 * mh + ((j & 3) >> 1)) ^ (2 * t)) + 4 * (j & 1));
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
  // r0 is a multiple of 16 and c0 of 32: row r0 + (8t + 4hh + j/4), column
  // c0 + 16mh + 4(j%4) is chunk 4*(c0/32) + (2mh + (j%4)/2), element 4(j%2)
  const int j = lane & 15, mh = (lane >> 4) & 1, hh = lane >> 5;
  s16x4 v[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int off = tile_off_split<D>(r0 + 8 * t, 4 * hh + (j >> 2), c0 >> 5, 2 * mh + ((j & 3) >> 1)) + 4 * (j & 1);
    v[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_ptr(tile) + off));
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
// A unit is `rep` consecutive items (longest-first order) times the grp
// q-heads of one kv-head, on consecutive slots of one XCD, so its workgroups
// start together and stream the same K/V tiles through that XCD's L2.  A
// GQA group of 4 or more q-heads already gives that sharing (rep = 1); with
// fewer (MHA) a unit takes several query tiles of the same head instead:
// on the teacher-forcing DiT shape (24 heads, MHA) this cut the forward's
// HBM fetch from 63 GB to 23 GB per launch and sped it up by ~4.5 %.
__host__ __device__ inline int items_per_unit(int grp) { return grp >= 4 ? 1 : (32 + grp - 1) / grp; }

__device__ __forceinline__ void map_block(int bid, int grp, int hkv, int& item_rank, int& head, int& kvh,
                                          int rep = 1) {
  const int x = bid & 7;
  const int k = bid >> 3;
  const int P = grp * rep;
  const int u = k / P, j = k - u * P;
  const int U = u * 8 + x;
  const int iu = U / hkv;
  kvh = U - iu * hkv;
  const int jr = j / grp;
  item_rank = iu * rep + jr;
  head = kvh * grp + (j - jr * grp);
}

inline unsigned unit_grid(int64_t max_items, int hkv, int grp, int rep = 1) {
  const int64_t units = (max_items + rep - 1) / rep * hkv;
  return (unsigned)(((units + 7) / 8) * 8 * grp * rep);
}

}  // namespace cpattn
