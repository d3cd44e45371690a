// Forward ring step: blockwise attention of the local queries against the
// K/V share held at this step ("Scaling Video Training with Parallelism",
// section 2, Ring Attention paragraph), with the online softmax that makes
// a block's output and log-sum-exp exact for that block.
//
// bf16 path (gfx950 MFMA).  One workgroup = one tile of 128 query rows x one
// q-head; 4 waves of 32 query rows each, compiled for two waves per SIMD
// (two workgroups per CU, 64 KiB of LDS each).  Per key tile of 64 rows:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS, Q in registers;
//                    the transposed product puts one query per lane column,
//                    so row statistics are in-lane plus one lane^32 swap.
//   mask             only on tiles the scheduler did not mark fully allowed.
//   online softmax   exp2 with log2(e) folded into the scale, fp32, with
//                    lazy rescaling of the running output.
//   O^T += V^T P^T   P rounded to bf16 straight from the accumulator
//                    registers; V^T operands come from the row-major V tile
//                    through transposing LDS reads (ds_read_b64_tr_b16).
// The tile loop is software-pipelined across tiles: the S^T products of
// tile j + 1 and the PV products of tile j carry tile j's softmax and tile
// j + 1's row max (see the kernel).  K and V tiles move global -> LDS with
// direct loads (no register staging), double-buffered with one barrier per
// tile.  Workgroups are mapped so that the q-heads of one GQA group and the
// tiles of one kv-head land on the same XCD, keeping their K/V in that
// XCD's L2.  Measured alternatives: 64 query rows per wave (one wave per
// SIMD) and per-32-key softmax blocks were slower.
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
constexpr int kFwdPF = CPATTN_FWD_PF;   // operand reads ahead of their products



// ---------------------------------------------------------------------------
// bf16 kernel, software-pipelined across key tiles (32 queries per wave,
// two waves per SIMD).  Iteration j issues the S^T products of tile j + 1 and the PV
// products of tile j, and spreads tile j's softmax over them:
//   S^T(j+1) products:  rescale decision of tile j, exp + pack of its key
//                       block 0, then exp of key block 1
//   PV(j) products:     rest of block 1's exp and its pack (before the block-1
//                       products need it), then mask and row max of tile j + 1
// K of tile j + 2 and V of tile j + 1 load during iteration j into the
// buffers that tiles j and j - 1 released, so one barrier per iteration and
// double buffering suffice.  Operand reads run PF products ahead; every
// product slot is fenced so the interleave holds.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BN = 64;
  constexpr int NK = D / 16;       // k-steps of one 32-key S^T block; PV products per 16-key k-step pair
  constexpr int NS = 2 * NK;       // S^T products per tile (two key blocks)
  constexpr int NP = 4 * (D / 32); // PV products per tile
  constexpr int PF = kFwdPF;
  // Four separate arrays (not one [2][..] array per operand): every buffer
  // index below is a compile-time constant, so the compiler can tell a read
  // of one buffer from the direct loads still filling the other and does
  // not wait for those loads before the read.
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[BN * D], s_k1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[BN * D], s_v1[BN * D];

  int item_rank, h, g;
  map_block(blockIdx.x, a.grp, a.hkv, item_rank, h, g, items_per_unit(a.grp));
  // the item count and the item's order entry load together (the entry is
  // read in bounds, and dropped for a rank past the count)
  const int n_items = a.hdr->n_items;
  const int oi = a.order[min(item_rank, a.order_cap - 1)];
  asm volatile("" ::"s"(oi), "s"(n_items));   // both loads issued before the test
  if (item_rank >= n_items) return;
  const WorkItem it = a.items[oi];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col = lane & 31, hh = lane >> 5;
  // lane parts of the K row reads (k-step parity 0, 1) and the V^T reads
  const int lko[2] = {opaque_lane(tile_off_lane<D>(col, hh)), opaque_lane(tile_off_lane<D>(col, 2 ^ hh))};
  int lvo[2];
  tr_lane_offsets<D>(lane, lvo);
  const int64_t kst = a.k_st * 2, vst = a.v_st * 2;
  const char* kbase = (const char*)a.k + (int64_t)g * a.k_sh * 2;
  const char* vbase = (const char*)a.v + (int64_t)g * a.v_sh * 2;
  TileLoader<D, BN, NW> lk, lv;
  lk.init(kst, wave, lane);
  lv.init(vst, wave, lane);

  const int nt0 = it.nseg > 0 ? ceil_div(it.seg[0].n, BN) : 0;
  const int nt1 = it.nseg > 1 ? ceil_div(it.seg[1].n, BN) : 0;
  const int ntiles = nt0 + nt1;
  auto tile_at = [&](int j, int& t0, Segment& sg) {
    const int s = j < nt0 ? 0 : 1;
    t0 = (j - (s ? nt0 : 0)) * BN;
    sg = it.seg[s];
  };
  // tile j goes to buffer j & 1; `buf` is that buffer (a constant at each call)
  auto issue_k = [&](int j, uint16_t* buf) {
    int t0;
    Segment sg;
    tile_at(j, t0, sg);
    lk.issue(buf, kbase + (int64_t)(sg.row + t0) * kst, min(BN, sg.n - t0), kst);
  };
  auto issue_v = [&](int j, uint16_t* buf) {
    int t0;
    Segment sg;
    tile_at(j, t0, sg);
    lv.issue(buf, vbase + (int64_t)(sg.row + t0) * vst, min(BN, sg.n - t0), vst);
  };
  const int r = wave * 32 + col;
  const bool row_ok = r < it.nrows;
  const KeyWindows kw = key_windows(key_ranges(a.mask, it.pos0 + r, a.tf_b, a.tf_n));
  bf16x8 qreg[NK];
  {
    const uint16_t* src = (const uint16_t*)a.q + (int64_t)(it.row0 + r) * a.q_st + (int64_t)h * a.q_sh + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = *(const u32x4*)(src + 16 * ks);
      qreg[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  // Q is loaded before the first K/V tiles, so the prologue's wait for
  // K(0) (vmcnt counts in issue order) also covers Q and leaves V(0) and
  // K(1) in flight; the fence keeps the compiler from sinking the Q loads.
  asm volatile("" ::: "memory");
  if (ntiles > 0) {
    issue_k(0, s_k0);
    issue_v(0, s_v0);
    if (ntiles > 1) issue_k(1, s_k1);
  }
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // S^T of one tile: two 32-key accumulator chains, key block 0 first.
  f32x16 sacc[2][2];     // [tile parity][key block]
  float smax[2];         // scaled row max of the tile held in sacc[parity]
  // mask of a partial tile, then its scaled row max
  auto mask_block = [&](f32x16 (&st)[2], int kb, int t0, const Segment& sg) {
    const int kbase0 = t0 + 32 * kb + 4 * hh;
    const unsigned bits = allowed_bits(kw, sg.pos + kbase0, sg.n - kbase0);
    for_each_index<16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      st[kb][i] = select_bit<8 * (i >> 2) + (i & 3)>(bits, st[kb][i], 0xff800000u);
    });
  };
  auto rowmax_part = [&](const f32x16& v, float m) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) m = max3f(m, v[i], v[i + 1]);
    return m;
  };

  // prologue: S^T of tile 0 with its mask and row max
  if (ntiles > 0) {
    wait_vmcnt_tiles<TileLoader<D, BN, NW>::PER>(ntiles > 1 ? 2 : 1);   // K(0) in; V(0), K(1) may load
    // a bare barrier: __syncthreads() would also wait for V(0) and K(1)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[0][kb][i] = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u)
      sacc[0][u / NK] = mfma32(read_row8_at<D>(s_k0, lko[(u % NK) & 1], 32 * (u / NK), u % NK), qreg[u % NK], sacc[0][u / NK]);
    int t0;
    Segment sg;
    tile_at(0, t0, sg);
    if (!(t0 >= sg.full_lo && t0 + BN <= sg.full_hi)) {
      mask_block(sacc[0], 0, t0, sg);
      mask_block(sacc[0], 1, t0, sg);
    }
    smax[0] = max_halves(rowmax_part(sacc[0][1], rowmax_part(sacc[0][0], -INFINITY))) * a.scale_log2;
  }

  // MORE: a tile j + 1 follows (compile-time, so the product slots carry no
  // branches on it)
  auto iter = [&](int j, auto parc, auto morec) {
    constexpr int P = decltype(parc)::value;       // j & 1: V(j) buffer, sacc/smax slot of tile j
    constexpr int Q = P ^ 1;                       // slot of tile j + 1
    constexpr bool more = decltype(morec)::value;
    wait_loads();                                  // K(j+1), V(j) in (issued an iteration ago)
    __syncthreads();
    if (j + 2 < ntiles) issue_k(j + 2, P ? s_k1 : s_k0);   // into K(j)'s buffer
    if (more) issue_v(j + 1, Q ? s_v1 : s_v0);             // into V(j-1)'s buffer
    const uint16_t* tk = Q ? s_k1 : s_k0;
    const uint16_t* tv = P ? s_v1 : s_v0;
    int t1 = 0;
    Segment sg1 = it.seg[0];
    if (more) tile_at(j + 1, t1, sg1);
    const bool full1 = t1 >= sg1.full_lo && t1 + BN <= sg1.full_hi;

    // ---- softmax of tile j, in slots -------------------------------------
    bf16x8 pb[4];
    float m_use = 0.f;
    auto rescale = [&]() {
      const float mt = smax[P];
      if (__any(mt > m_run + kRescale)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
      }
      m_use = m_run == -INFINITY ? 0.f : m_run;
    };
    auto exps = [&](int kb, int i0, int i1) {
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[P][kb][i] * a.scale_log2 - m_use);
        sacc[P][kb][i] = p;
        l_run += p;
      }
    };
    auto pack = [&](int kb) {
      pb[2 * kb] = pack_b(sacc[P][kb], 0);
      pb[2 * kb + 1] = pack_b(sacc[P][kb], 1);
      asm volatile("" : "+v"(pb[2 * kb]), "+v"(pb[2 * kb + 1]));
    };
    float mx1 = -INFINITY;
    // work of slot `sl` (0 .. NS + NP - 1): S^T(j+1) products come first
    // Slot s carries its work after its product.  Block 0's pack lands in the
    // S^T slots (before PV product 0); block 1's before PV product NP/2,
    // the first one that reads it.
    constexpr int EA = NS / 2 - 1;                 // slots 1..EA: block-0 exps; EA+1: its pack
    constexpr int B0 = EA + 2, B1 = NS + NP / 2 - 2;   // [B0, B1): block-1 exps; B1: its pack
    static_assert(EA + 1 < NS && B1 < NS + NP / 2 && B1 > B0, "packs precede their PV products");
    auto slot_work = [&](int sl) {
      if (sl == 0) rescale();
      if (sl >= 1 && sl <= EA) exps(0, (sl - 1) * 16 / EA, sl * 16 / EA);
      if (sl == EA + 1) pack(0);
      if (sl >= B0 && sl < B1) exps(1, (sl - B0) * 16 / (B1 - B0), (sl - B0 + 1) * 16 / (B1 - B0));
      if (sl == B1) pack(1);
      if (more) {
        if (sl == NS + NP / 2 && !full1) { mask_block(sacc[Q], 0, t1, sg1); mask_block(sacc[Q], 1, t1, sg1); }
        if (sl == NS + NP / 2 + 1) mx1 = rowmax_part(sacc[Q][0], -INFINITY);
        if (sl == NS + NP / 2 + 2) smax[Q] = max_halves(rowmax_part(sacc[Q][1], mx1)) * a.scale_log2;
      }
    };

    // ---- products ----------------------------------------------------------
    bf16x8 kop[NS], vop[NP];
    auto read_k = [&](int u) { kop[u] = read_row8_at<D>(tk, lko[(u % NK) & 1], 32 * (u / NK), u % NK); };
    auto read_v = [&](int m) {          // PV product m: k-step pair ps = m / (D/32), d-block m % (D/32)
      vop[m] = read_tr_at<D>(tv, lvo, 16 * (m / (D / 32)), 32 * (m % (D / 32)));
    };
    auto read_op = [&](int x) {         // operand x of the iteration's product sequence
      if (x < NS) { if (more) read_k(x); }
      else read_v(x - NS);
    };
    if (more) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[Q][kb][i] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < PF; ++x) read_op(more ? x : NS + x);
    // Wave priority: the PV half of an iteration (whose second half carries
    // the mask and row max of tile j + 1) issues ahead of a co-resident
    // wave's S^T half (measured: +1 to +3 % over equal priority).
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (more) {
        if (u + PF < NS + NP) read_op(u + PF);
        sacc[Q][u / NK] = mfma32(kop[u], qreg[u % NK], sacc[Q][u / NK]);
      }
      slot_work(u);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      if (m + PF < NP) read_v(m + PF);
      acc_o[m % (D / 32)] = mfma32(vop[m], pb[m / (D / 32)], acc_o[m % (D / 32)]);
      slot_work(NS + m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  int j = 0;
  for (; j + 2 < ntiles; j += 2) {
    iter(j, I0{}, T{});
    iter(j + 1, I1{}, T{});
  }
  if (j + 1 < ntiles) {
    iter(j, I0{}, T{});
    iter(j + 1, I1{}, F{});
  } else if (j < ntiles) {
    iter(j, I0{}, F{});
  }

  const float l = sum_halves(l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  // O leaves through LDS so that every store writes whole rows: each wave
  // puts its 32 rows into a block of its own, 16-byte chunks swizzled by row
  // (conflict-free writes down a column), and reads them back row-major.
  // The K buffers are free here: the last iteration reads only V, and all
  // waves passed its barrier after their last K read.
  // (The lane index is recomputed here rather than kept live through the
  // tile loop, where the register file is full.)
  const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int ecol = ln & 31, ehh = ln >> 5;
  {
    constexpr int CH = D / 8;                                // 16-byte chunks per row
    constexpr int RPI = 64 / CH;                             // rows per read instruction
    char* blk = (char*)((wave < 2 ? s_k0 : s_k1) + (wave & 1) * 32 * D);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc_o[db][4 * i4 + e] * inv);
        const int chunk = db * 4 + i4;
        *(u32x2*)(blk + ecol * (2 * D) + ((chunk ^ (ecol & (CH - 1))) << 4) + 8 * ehh) = __builtin_bit_cast(u32x2, w);
      }
    const int rl = ln / CH, ch = ln % CH;
    u32x4 v[32 / RPI];
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int rr = k * RPI + rl;                           // row within the wave's 32
      v[k] = *(const u32x4*)(blk + rr * (2 * D) + ((ch ^ (rr & (CH - 1))) << 4));
    }
    uint16_t* orow = (uint16_t*)a.out + (int64_t)(it.row0 + wave * 32 + rl) * a.o_st + (int64_t)h * a.o_sh + 8 * ch;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k)
      if (wave * 32 + k * RPI + rl < it.nrows) *(u32x4*)(orow + (int64_t)(k * RPI) * a.o_st) = v[k];
  }
  if (ehh == 0 && wave * 32 + ecol < it.nrows)
    a.lse[(int64_t)h * a.tq + it.row0 + wave * 32 + ecol] =
        l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
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

#ifndef CPATTN_FWD_WAVES
#define CPATTN_FWD_WAVES 4
#endif
constexpr int kFwdWaves = CPATTN_FWD_WAVES;
constexpr int kFwdTile = 32 * kFwdWaves;   // query rows per workgroup

int fwd_tile_rows(bool bf16) { return bf16 ? kFwdTile : 64; }

hipError_t launch_fwd(const FwdArgs& a0, bool bf16, int d, int64_t max_items, hipStream_t stream) {
  FwdArgs a = a0;
  a.order_cap = (int)max_items;
  const dim3 grid(unit_grid(max_items, a.hkv, a.grp, bf16 ? items_per_unit(a.grp) : 1));
  if (bf16) {
    if (d == 128) hipLaunchKernelGGL((fwd_bf16_kernel<128, kFwdWaves>), grid, dim3(64 * kFwdWaves), 0, stream, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, kFwdWaves>), grid, dim3(64 * kFwdWaves), 0, stream, a);
  } else {
    if (d == 128) hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cpattn
