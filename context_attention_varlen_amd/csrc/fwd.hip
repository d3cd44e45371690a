// Forward ring step: blockwise attention of the local queries against the
// K/V share held at this step ("Scaling Video Training with Parallelism",
// section 2, Ring Attention paragraph), with the online softmax that makes
// a block's output and log-sum-exp exact for that block.
//
// bf16 path (gfx950 MFMA).  One workgroup = one tile of 128 query rows x one
// q-head; 4 waves of 32 query rows each, compiled for two waves per SIMD
// (two workgroups per CU, 64 KiB of LDS each), so that one wave's softmax
// runs while the other's MFMAs do (with one wave per SIMD the MFMA drains,
// cross-lane exchanges and barriers stall the SIMD).  The kernel is also
// templated for 64 query rows per wave (two MFMA column blocks sharing every
// K operand read); that form needs one wave per SIMD and measured slower.
// Per key tile of 64 rows:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS, Q in registers;
//                    the transposed product puts one query per lane column,
//                    so row statistics are in-lane plus one lane^32 swap.
//   mask             only on tiles the scheduler did not mark fully allowed.
//   online softmax   exp2 with log2(e) folded into the scale, fp32, with
//                    lazy rescaling of the running output.
//   O^T += V^T P^T   P rounded to bf16 straight from the accumulator
//                    registers; V^T operands come from the row-major V tile
//                    through transposing LDS reads (ds_read_b64_tr_b16).
// K and V tiles move global -> LDS with direct loads (no register staging),
// double-buffered with one barrier per tile; the next tile's loads are in
// flight during the current tile's math.  Workgroups are mapped so that the
// q-heads of one GQA group and the tiles of one kv-head land on the same XCD,
// keeping their K/V in that XCD's L2.
//
// fp32 path: a plain per-row kernel (one query row per thread, exact expf)
// for fp32 inputs; it exists for accuracy checks, not speed.
#include <type_traits>

#include "mfma.h"

namespace cpattn {


// Lazy rescaling: the running max m only moves when a tile's max exceeds it
// by more than kRescale (log2 units), so P = exp2(s - m) stays <= 2^8 and
// the O rescale (D/32 x 16 multiplies per query block) is skipped on most
// tiles.  O / l and m + log2(l) use the same m, so the result is exact.
constexpr float kRescale = 8.0f;

#ifndef CPATTN_FWD_PF
#define CPATTN_FWD_PF 3
#endif
constexpr int kFwdPF = CPATTN_FWD_PF;   // K operand reads ahead of their products



// Waves per SIMD the kernel is compiled for: two when each wave owns 32
// queries (so one wave's softmax overlaps the other's MFMAs), else one.
template <int QB>
struct FwdOcc { static constexpr int value = QB == 1 ? 2 : 1; };

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FwdOcc<QB>::value, FwdOcc<QB>::value)))
void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BN = 64;
  constexpr int QW = 32 * QB;                 // query rows per wave
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][BN * D];

  int item_rank, h, g;
  map_block(blockIdx.x, a.grp, a.hkv, item_rank, h, g);
  if (item_rank >= a.hdr->n_items) return;
  const WorkItem it = a.items[a.order[item_rank]];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col = lane & 31, hh = lane >> 5;

  const int64_t kst = a.k_st * 2, vst = a.v_st * 2;     // row strides in bytes
  const char* kbase = (const char*)a.k + (int64_t)g * a.k_sh * 2;
  const char* vbase = (const char*)a.v + (int64_t)g * a.v_sh * 2;
  TileLoader<D, BN, NW> lk, lv;
  lk.init(kst, wave, lane);
  lv.init(vst, wave, lane);

  const int nt0 = it.nseg > 0 ? ceil_div(it.seg[0].n, BN) : 0;
  const int nt1 = it.nseg > 1 ? ceil_div(it.seg[1].n, BN) : 0;
  const int ntiles = nt0 + nt1;
  auto issue = [&](int j, int buf) {
    const int s = j < nt0 ? 0 : 1;
    const int t0 = (j - (s ? nt0 : 0)) * BN;
    const Segment& sg = it.seg[s];
    const int nvalid = min(BN, sg.n - t0);
    const int64_t row = sg.row + t0;
    lk.issue(s_k[buf], kbase + row * kst, nvalid, kst);
    lv.issue(s_v[buf], vbase + row * vst, nvalid, vst);
  };
  if (ntiles > 0) issue(0, 0);

  // Q operand (B of S^T = K Q^T): lane holds Q[row][16*ks + 8*hh + 0..7]
  bf16x8 qreg[QB][D / 16];
  KeyRanges kr[QB];
  bool row_ok[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = wave * QW + qb * 32 + col;
    row_ok[qb] = r < it.nrows;
    kr[qb] = key_ranges(a.mask, it.pos0 + r, a.tf_b, a.tf_n);
    const uint16_t* src = (const uint16_t*)a.q + (int64_t)(it.row0 + r) * a.q_st + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok[qb]) raw = *(const u32x4*)(src + 16 * ks);
      qreg[qb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 acc_o[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[qb][db][i] = 0.f;
  }

  // One key tile; BUF is a compile-time buffer index so every LDS offset is
  // an immediate.
  auto tile = [&](int j, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_loads();
    __syncthreads();
    if (j + 1 < ntiles) issue(j + 1, buf ^ 1);
    const int s = j < nt0 ? 0 : 1;
    const int t0 = (j - (s ? nt0 : 0)) * BN;
    const Segment sg = it.seg[s];
    const uint16_t* tk = s_k[buf];
    const uint16_t* tv = s_v[buf];
    const bool full = t0 >= sg.full_lo && t0 + BN <= sg.full_hi;
    // S^T for the whole 64-key tile, then one softmax update, then PV. The
    // two 32-key blocks of S^T run as one accumulator chain each, block 0
    // first, so block 0's mask and partial row max are done under block 1's
    // products. K operands are read PF products ahead; each step is fenced.
    static_assert(QB == 1 && BN == 64, "the tile schedule covers one 32-query block and two key blocks");
    constexpr int NK = D / 16;
    f32x16 acc_s[QB][BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_s[0][kb][i] = 0.f;
    auto mask_block = [&](int kb) {
      if (!full) {
        const int kbase0 = t0 + kb * 32 + 4 * hh;     // key offset of register 0
        const int rem = sg.n - kbase0;                 // registers at offset >= rem are past the segment
        const int pbase = sg.pos + kbase0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 8 * (i >> 2) + (i & 3);
          acc_s[0][kb][i] = ((off < rem) & in_ranges(kr[0], pbase + off)) ? acc_s[0][kb][i] : -INFINITY;
        }
      }
    };
    bf16x8 kop[2 * NK];
    auto read_k = [&](int u) { kop[u] = read_row8<D>(tk, 32 * (u / NK), col, u % NK, hh); };
#pragma unroll
    for (int u = 0; u < kFwdPF; ++u) read_k(u);
    float mx0 = 0.f;
#pragma unroll
    for (int u = 0; u < 2 * NK; ++u) {
      if (u + kFwdPF < 2 * NK) read_k(u + kFwdPF);
      acc_s[0][u / NK] = mfma32(kop[u], qreg[0][u % NK], acc_s[0][u / NK]);
      if (u == NK + 2) mask_block(0);
      if (u == NK + 3)
        mx0 = max3f(max3f(max3f(max3f(acc_s[0][0][0], acc_s[0][0][1], acc_s[0][0][2]), acc_s[0][0][3], acc_s[0][0][4]),
                          acc_s[0][0][5], acc_s[0][0][6]), acc_s[0][0][7], acc_s[0][0][8]);
      if (u == NK + 4)
        mx0 = fmaxf(max3f(max3f(max3f(mx0, acc_s[0][0][9], acc_s[0][0][10]), acc_s[0][0][11], acc_s[0][0][12]),
                          acc_s[0][0][13], acc_s[0][0][14]), acc_s[0][0][15]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NK + 2 >= 2 * NK) mask_block(0);   // D = 64: block 1 is too short to carry them
    if (NK + 3 >= 2 * NK)
      mx0 = max3f(max3f(max3f(max3f(acc_s[0][0][0], acc_s[0][0][1], acc_s[0][0][2]), acc_s[0][0][3], acc_s[0][0][4]),
                        acc_s[0][0][5], acc_s[0][0][6]), acc_s[0][0][7], acc_s[0][0][8]);
    if (NK + 4 >= 2 * NK)
      mx0 = fmaxf(max3f(max3f(max3f(mx0, acc_s[0][0][9], acc_s[0][0][10]), acc_s[0][0][11], acc_s[0][0][12]),
                        acc_s[0][0][13], acc_s[0][0][14]), acc_s[0][0][15]);
    mask_block(1);
    float mt[QB];
    bool need = false;
    {
      float mx = mx0;
#pragma unroll
      for (int i = 0; i + 1 < 16; i += 2) mx = max3f(mx, acc_s[0][1][i], acc_s[0][1][i + 1]);
      mt[0] = max_halves(mx) * a.scale_log2;
      need |= mt[0] > m_run[0] + kRescale;
    }
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_run[qb], mt[qb]);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[qb][db][i] *= alpha;
      }
    }
    bf16x8 pb[QB][BN / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(acc_s[qb][kb][i] * a.scale_log2 - m_use);
          acc_s[qb][kb][i] = p;
          l_run[qb] += p;
        }
        pb[qb][2 * kb] = pack_b(acc_s[qb][kb], 0);
        pb[qb][2 * kb + 1] = pack_b(acc_s[qb][kb], 1);
      }
    }
    // consecutive MFMAs go to different accumulators (independent chains)
#pragma unroll
    for (int ps = 0; ps < BN / 16; ++ps)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 av = read_tr<D>(tv, 16 * ps, 32 * db, lane);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc_o[qb][db] = mfma32(av, pb[qb][ps], acc_o[qb][db]);
      }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, std::integral_constant<int, 0>{});
    if (j + 1 < ntiles) tile(j + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = sum_halves(l_run[qb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (!row_ok[qb]) continue;
    const int r = wave * QW + qb * 32 + col;
    uint16_t* op = (uint16_t*)a.out + (int64_t)(it.row0 + r) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc_o[qb][db][4 * i4 + e] * inv);
        *(u32x2*)(op + db * 32 + 8 * i4 + 4 * hh) = __builtin_bit_cast(u32x2, w);
      }
    if (hh == 0)
      a.lse[(int64_t)h * a.tq + it.row0 + r] =
          l > 0.f ? (m_run[qb] + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
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

#ifndef CPATTN_FWD_QB
#define CPATTN_FWD_QB 1
#endif

#ifndef CPATTN_FWD_WAVES
#define CPATTN_FWD_WAVES 4
#endif
constexpr int kFwdWaves = CPATTN_FWD_WAVES, kFwdQB = CPATTN_FWD_QB;
constexpr int kFwdTile = 32 * kFwdQB * kFwdWaves;

int fwd_tile_rows(bool bf16) { return bf16 ? kFwdTile : 64; }

hipError_t launch_fwd(const FwdArgs& a, bool bf16, int d, int64_t max_items, hipStream_t stream) {
  const dim3 grid(unit_grid(max_items, a.hkv, a.grp));
  if (bf16) {
    if (d == 128) hipLaunchKernelGGL((fwd_bf16_kernel<128, kFwdWaves, kFwdQB>), grid, dim3(64 * kFwdWaves), 0, stream, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, kFwdWaves, kFwdQB>), grid, dim3(64 * kFwdWaves), 0, stream, a);
  } else {
    if (d == 128) hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cpattn
