// Forward ring step: blockwise attention of the local queries against the
// K/V share held at this step ("Scaling Video Training with Parallelism",
// section 2, Ring Attention paragraph), with the online softmax that makes
// a block's output and log-sum-exp exact for that block.
//
// bf16 path (gfx950 MFMA).  One workgroup = one query tile of 128 rows x one
// q-head; 4 waves, each owning 32 query rows.  Per key tile of 64 rows:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS, Q in registers;
//                    the transposed product puts one query per lane column,
//                    so row statistics are in-lane plus one lane^32 swap.
//   mask             only on tiles the scheduler did not mark fully allowed.
//   online softmax   exp2 with log2(e) folded into the scale, fp32.
//   O^T += V^T P^T   P rounded to bf16 straight from the accumulator
//                    registers; V is stored transposed in LDS with its key
//                    order permuted to match the accumulator layout.
// K and V^T tiles are double-buffered in LDS (one barrier per tile) and the
// next tile's global loads are in flight during the current tile's math.
// Workgroups are mapped so that the q-heads of one GQA group and the tiles
// of one kv-head land on the same XCD (dispatch is round-robin over 8 XCDs),
// keeping their K/V in that XCD's L2.
//
// fp32 path: a plain per-row kernel (one query row per thread, exact expf)
// for fp32 inputs; it exists for accuracy checks, not speed.
#include "common.h"

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));



// blockIdx -> (item rank, q-head).  Consecutive dispatch slots of one XCD
// (bid % 8) take the G q-heads of one (item, kv-head) unit; units are dealt
// round-robin to XCDs in item order, so with Hkv dividing 8 (or 8 dividing
// Hkv) each XCD keeps to a fixed set of kv-heads.
__device__ __forceinline__ void map_block(int bid, int grp, int hkv, int& item_rank, int& head, int& kvh) {
  const int x = bid & 7;
  const int k = bid >> 3;
  const int u = k / grp, j = k - u * grp;
  const int U = u * 8 + x;
  item_rank = U / hkv;
  kvh = U - item_rank * hkv;
  head = kvh * grp + j;
}

__device__ __forceinline__ int swap23(int x) { return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int D>
struct FwdCfg {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int KCH = D / 8;               // 16-byte chunks per K row
  static constexpr int LOADS = BN * KCH / NT;     // chunks per thread per tile
  static constexpr int K_ELEMS = BN * D;          // one K (or V^T) buffer
};

// V^T element offset in LDS: row d holds BN keys at permuted positions,
// 16-byte chunks XOR-swizzled by (d + d/8) % 8.
template <int BN>
__device__ __forceinline__ int vt_off(int d, int pos) {
  const int ch = (pos >> 3) ^ ((d + (d >> 3)) & 7);
  return d * BN + ch * 8 + (pos & 7);
}

template <int D>
__device__ __forceinline__ int k_off(int row, int ch) {
  return row * D + ((ch ^ (row & (D / 8 - 1))) << 3);
}

template <int D>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][C::K_ELEMS];

  int item_rank, h, g;
  map_block(blockIdx.x, a.grp, a.hkv, item_rank, h, g);
  if (item_rank >= a.hdr->n_items) return;
  const WorkItem it = a.items[a.order[item_rank]];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int qrow = wave * 32 + col;                 // row in the tile
  const bool row_ok = qrow < it.nrows;
  const int pq = it.pos0 + qrow;

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k;
  const uint16_t* vp = (const uint16_t*)a.v;

  // Q operand: lane holds Q[qrow][16*ks + 8*hh + 0..7]
  bf16x8 qreg[D / 16];
  {
    const uint16_t* src = qp + (int64_t)(it.row0 + qrow) * a.q_st + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = *(const u32x4*)(src + 16 * ks);
      qreg[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 acc_o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nt0 = it.nseg > 0 ? ceil_div(it.seg[0].n, BN) : 0;
  const int nt1 = it.nseg > 1 ? ceil_div(it.seg[1].n, BN) : 0;
  const int ntiles = nt0 + nt1;

  const uint16_t* kbase = kp + (int64_t)g * a.k_sh;
  const uint16_t* vbase = vp + (int64_t)g * a.v_sh;

  u32x4 pk[C::LOADS], pv[C::LOADS];
  auto tile_of = [&](int j, int& s, int& t0) {
    s = j < nt0 ? 0 : 1;
    t0 = (j - (s ? nt0 : 0)) * BN;
  };
  auto gload = [&](int j) {
    int s, t0;
    tile_of(j, s, t0);
    const int srow = it.seg[s].row, sn = it.seg[s].n;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / C::KCH, ch = c - r * C::KCH;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (t0 + r < sn) {
        const int64_t row = srow + t0 + r;
        zk = *(const u32x4*)(kbase + row * a.k_st + ch * 8);
        zv = *(const u32x4*)(vbase + row * a.v_st + ch * 8);
      }
      pk[i] = zk;
      pv[i] = zv;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / C::KCH, ch = c - r * C::KCH;
      *(u32x4*)(&s_k[buf][k_off<D>(r, ch)]) = pk[i];
      const int pos = swap23(r);
      const uint16_t* e = (const uint16_t*)&pv[i];
#pragma unroll
      for (int x = 0; x < 8; ++x) s_vt[buf][vt_off<BN>(ch * 8 + x, pos)] = e[x];
    }
  };

  if (ntiles > 0) gload(0);
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    lstore(buf);
    __syncthreads();
    int s, t0;
    tile_of(j, s, t0);
    if (j + 1 < ntiles) gload(j + 1);

    // ---- S^T = K Q^T ----
    f32x16 acc_s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_s[kb][i] = 0.f;
      const int krow = kb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)(&s_k[buf][k_off<D>(krow, 2 * ks + hh)]));
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[ks], acc_s[kb], 0, 0, 0);
      }
    }

    // ---- mask (partial tiles only) ----
    const Segment sg = it.seg[s];
    const bool full = t0 >= sg.full_lo && t0 + BN <= sg.full_hi;
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kofs = t0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool ok = kofs < sg.n && mask_allowed(a.mask, pq, sg.pos + kofs, a.tf_b, a.tf_n);
          if (!ok) acc_s[kb][i] = -INFINITY;
        }
    }

    // ---- online softmax ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc_s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;

    bf16x8 pb[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(acc_s[kb][i] * a.scale_log2 - m_use);
        l_run += p;
        pb[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
      }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int ps = 0; ps < BN / 16; ++ps) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)(&s_vt[buf][vt_off<BN>(d, 16 * ps + 8 * hh)]));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ps], acc_o[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue ----
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (row_ok) {
    uint16_t* op = (uint16_t*)a.out + (int64_t)(it.row0 + qrow) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc_o[db][4 * i4 + e] * inv);
        *(u32x2*)(op + db * 32 + 8 * i4 + 4 * hh) = __builtin_bit_cast(u32x2, w);
      }
    if (hh == 0)
      a.lse[(int64_t)h * a.tq + it.row0 + qrow] =
          l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one query row per thread, keys read from global memory.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
  int item_rank, h, g;
  map_block(blockIdx.x, a.grp, a.hkv, item_rank, h, g);
  if (item_rank >= a.hdr->n_items) return;
  const WorkItem it = a.items[a.order[item_rank]];
  const int r = threadIdx.x;
  const bool row_ok = r < it.nrows;
  const int pq = it.pos0 + r;
  const float* qp = (const float*)a.q + (int64_t)(it.row0 + (row_ok ? r : 0)) * a.q_st + (int64_t)h * a.q_sh;
  float qv[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { qv[c] = row_ok ? qp[c] : 0.f; o[c] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int s = 0; s < it.nseg; ++s) {
    const Segment sg = it.seg[s];
    for (int kk = 0; kk < sg.n; ++kk) {
      const bool ok = (kk >= sg.full_lo && kk < sg.full_hi) ||
                      mask_allowed(a.mask, pq, sg.pos + kk, a.tf_b, a.tf_n);
      if (!ok) continue;
      const float* kr = (const float*)a.k + (int64_t)(sg.row + kk) * a.k_st + (int64_t)g * a.k_sh;
      const float* vr = (const float*)a.v + (int64_t)(sg.row + kk) * a.v_st + (int64_t)g * a.v_sh;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], kr[c], dot);
      const float sc = dot * a.scale;
      const float mn = fmaxf(m, sc);
      const float al = expf(m - mn);
      const float p = expf(sc - mn);
      l = l * al + p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, vr[c], o[c] * al);
      m = mn;
    }
  }
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = (float*)a.out + (int64_t)(it.row0 + r) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
  for (int c = 0; c < D; ++c) op[c] = o[c] * inv;
  a.lse[(int64_t)h * a.tq + it.row0 + r] = l > 0.f ? m + logf(l) : -INFINITY;
}

// Grid size for a work list of up to max_items items.
inline unsigned fwd_grid(int64_t max_items, int hkv, int grp) {
  const int64_t units = max_items * hkv;
  return (unsigned)(((units + 7) / 8) * 8 * grp);
}

hipError_t launch_fwd(const FwdArgs& a, bool bf16, int d, int64_t max_items, hipStream_t stream) {
  const dim3 grid(fwd_grid(max_items, a.hkv, a.grp));
  if (bf16) {
    if (d == 128) hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, dim3(256), 0, stream, a);
  } else {
    if (d == 128) hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cpattn
