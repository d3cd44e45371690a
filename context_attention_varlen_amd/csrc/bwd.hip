// Backward ring step, recomputing P from the final merged log-sum-exp.
//
// For the loss sum_i <dO_i, O_i>, with P_ij = exp(scale <q_i, k_j> - LSE_i)
// and delta_i = <dO_i, O_i> (final O):
//   dS_ij = P_ij (<dO_i, v_j> - delta_i)
//   dQ_i += scale sum_j dS_ij k_j,  dK_j += scale sum_i dS_ij q_i,
//   dV_j += sum_i P_ij dO_i
// with j over the keys of the K/V share held at this ring step.  Training
// through the ring ("Scaling Video Training with Parallelism", section 1:
// splitting must not change the loss) needs exactly these per-step pieces;
// the ring returns dK/dV of step s to their owner.
//
// One kernel launch per step with two kinds of workgroups, no atomics,
// deterministic:
//   dkv  one workgroup per (128-key tile, kv-head): 4 waves x 32 keys hold
//        K as an MFMA operand and dK^T, dV^T accumulators in registers (V's
//        operand rows are read from an LDS copy of the key tile), and sweep
//        every q-head of the GQA group and every query tile that can see the
//        keys (32 rows, Q/dO tiles in LDS, double-buffered):
//          S = Q K^T, dP = dO V^T               (row reads of Q, dO, V)
//          dV^T += dO^T P, dK^T += Q^T dS       (transposing reads of dO, Q)
//   dq   one workgroup per (128-query tile, q-head): 4 waves x 32 queries
//        hold Q, dO operands and dQ^T accumulators, sweeping key tiles:
//          S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T
// Each accumulator element is owned by one workgroup, so += is a plain
// read-modify-write.  Both kinds fit 256 registers per wave and ~65 KiB of
// LDS, so the kernel runs two waves per SIMD (two workgroups per CU).  The
// fp32 path uses plain per-row kernels.
#include <type_traits>

#include "mfma.h"

namespace cpattn {

namespace {

constexpr int kDqWaves = 4, kDqQB = 1;            // dq: 4 waves x 32 queries
constexpr int kDkvWaves = 4;                       // dkv: 4 waves x 32 keys
constexpr int kBwdBQ = 32;                         // query rows per LDS tile (dkv)
constexpr int kBwdBK = 64;                         // key rows per LDS tile (dq)
#ifndef CPATTN_DKV_PF
#define CPATTN_DKV_PF 2
#endif
#ifndef CPATTN_DKV_TPF
#define CPATTN_DKV_TPF 2
#endif
#ifndef CPATTN_DQ_PF
#define CPATTN_DQ_PF 2
#endif
constexpr int kDqPF = CPATTN_DQ_PF;                 // dq: operand reads ahead (products)
constexpr int kDkvPF = CPATTN_DKV_PF;               // dkv: S/dP operand reads ahead (k-steps)
constexpr int kDkvTPF = CPATTN_DKV_TPF;             // dkv: dV/dK transposed reads ahead (products)

// ---------------------------------------------------------------------------
// dq kernel (bf16)
// ---------------------------------------------------------------------------
template <int D, int NW, int QB>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a, int bid, uint16_t* smem) {
  constexpr int BN = kBwdBK;
  constexpr int QW = 32 * QB;
  uint16_t (*s_k)[BN * D] = (uint16_t (*)[BN * D])smem;
  uint16_t (*s_v)[BN * D] = (uint16_t (*)[BN * D])(smem + 2 * BN * D);

  int item_rank, h, g;
  map_block(bid, a.grp, a.hkv, item_rank, h, g, items_per_unit(a.grp));
  if (item_rank >= a.hdr_q->n_items) return;
  const WorkItem it = a.items_q[a.order_q[item_rank]];
  if (it.nseg == 0) return;

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col = lane & 31, hh = lane >> 5;
  const int64_t kst = a.k_st * 2, vst = a.v_st * 2;     // row strides in bytes
  const char* kbase = (const char*)a.k + (int64_t)g * a.k_sh * 2;
  const char* vbase = (const char*)a.v + (int64_t)g * a.v_sh * 2;
  TileLoader<D, BN, NW> lk, lv;
  lk.init(kst, wave, lane);
  lv.init(vst, wave, lane);

  const int nt0 = ceil_div(it.seg[0].n, BN);
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
  issue(0, 0);

  bf16x8 qreg[QB][D / 16], doreg[QB][D / 16];
  KeyRanges kr[QB];
  bool row_ok[QB];
  float lse2[QB], dlt[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = wave * QW + qb * 32 + col;
    row_ok[qb] = r < it.nrows;
    kr[qb] = key_ranges(a.mask, it.pos0 + r, a.tf_b, a.tf_n);
    const int64_t row = it.row0 + r;
    const uint16_t* qs = (const uint16_t*)a.q + row * a.q_st + (int64_t)h * a.q_sh + 8 * hh;
    const uint16_t* ds = (const uint16_t*)a.dout + row * a.do_st + (int64_t)h * a.do_sh + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 rq = {0u, 0u, 0u, 0u}, rd = {0u, 0u, 0u, 0u};
      if (row_ok[qb]) {
        rq = *(const u32x4*)(qs + 16 * ks);
        rd = *(const u32x4*)(ds + 16 * ks);
      }
      qreg[qb][ks] = __builtin_bit_cast(bf16x8, rq);
      doreg[qb][ks] = __builtin_bit_cast(bf16x8, rd);
    }
    float l = row_ok[qb] ? a.lse[(int64_t)h * a.tq + row] : -INFINITY;
    lse2[qb] = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;   // P = 0 for rows with no key
    dlt[qb] = row_ok[qb] ? a.delta[(int64_t)h * a.tq + row] : 0.f;
  }

  f32x16 acc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qb][db][i] = 0.f;

  static_assert(QB == 1 && BN == 64, "the dQ tile schedule covers one 32-query block and two 32-key blocks");
  constexpr int NK = D / 16;   // k-steps of S^T and dP^T; also dQ products per key block
  constexpr int PF = kDqPF;
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

    // Hand-pipelined tile of 64 keys (key blocks 0, 1) x this wave's 32
    // queries. Products in order: S0^T, dP0^T, S1^T, dP1^T (NK each, one
    // accumulator chain each; S^T = K Q^T, dP^T = V dO^T), then dQ0^T and
    // dQ1^T (dQ^T += K^T dS^T). VALU work rides under the products:
    // exp(S0) under dP0, dS0 under S1, exp(S1) under dP1, dS1 under dQ0.
    // Operands are read PF products ahead; every step is fenced. Element i
    // of a lane holds key 8*(i/4) + 4*hh + i%4 of its block, query `col`.
    f32x16 st[2], dpt[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) { st[b][i] = 0.f; dpt[b][i] = 0.f; }
    bf16x8 op[6 * NK];
    auto read_op = [&](int u) {
      if (u < 4 * NK) {  // row operand: block u / NK is S0, dP0, S1, dP1
        const int blk = u / NK, ks = u % NK;
        op[u] = read_row8<D>((blk & 1) ? tv : tk, 32 * (blk >> 1), col, ks, hh);
      } else {           // transposed K operand of dQ product m of key block kb
        const int kb = (u - 4 * NK) / NK, m = (u - 4 * NK) % NK;
        op[u] = read_tr<D>(tk, 32 * kb + 16 * (m & 1), 32 * (m >> 1), lane);
      }
    };
    auto exp_group = [&](int b, int g4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = __builtin_amdgcn_exp2f(st[b][4 * g4 + e] * a.scale_log2 - lse2[0]);
        asm("" : "+v"(pv));  // opaque to folds: the exp stays ahead of the mask branch
        st[b][4 * g4 + e] = pv;
      }
    };
    auto mask_block = [&](int b) {
      if (!full) {
        const int kb0 = t0 + b * 32 + 4 * hh;
        const int rem = sg.n - kb0;
        const int pbase = sg.pos + kb0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 8 * (i >> 2) + (i & 3);
          st[b][i] = ((off < rem) & in_ranges(kr[0], pbase + off)) ? st[b][i] : 0.f;
        }
      }
    };
    bf16x8 dsb[2][2];
    auto ds_group = [&](int b, int g4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) st[b][4 * g4 + e] = st[b][4 * g4 + e] * (dpt[b][4 * g4 + e] - dlt[0]);
    };
    // VALU riding under product ks of a phase: four groups from step 1 (dS)
    // or 2 (exp) on, the packs after them; what does not fit (D = 64) follows
    // the phase
    auto under_exp = [&](int b, int ks) { if (ks >= 2 && ks < 6) exp_group(b, ks - 2); };
    auto tail_exp = [&](int b) {
#pragma unroll
      for (int g4 = NK - 2; g4 < 4; ++g4) exp_group(b, g4);
    };
    // the packed dS is pinned where it is formed: it is used only after the
    // next mask branch, and would otherwise be sunk past it
    auto pack_ds = [&](int b, int hf) {
      dsb[b][hf] = pack_b(st[b], hf);
      asm volatile("" : "+v"(dsb[b][hf]));
    };
    auto under_ds = [&](int b, int ks) {
      if (ks >= 1 && ks < 5) ds_group(b, ks - 1);
      if (ks == 3) pack_ds(b, 0);
      if (ks == 5) pack_ds(b, 1);
    };
    auto tail_ds = [&](int b) {
#pragma unroll
      for (int g4 = NK - 1; g4 < 4; ++g4) ds_group(b, g4);
      if (3 >= NK) pack_ds(b, 0);
      if (5 >= NK) pack_ds(b, 1);
    };

#pragma unroll
    for (int u = 0; u < PF; ++u) read_op(u);
    auto step = [&](int u) { if (u + PF < 6 * NK) read_op(u + PF); };
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {           // S0^T
      step(ks);
      st[0] = mfma32(op[ks], qreg[0][ks], st[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {           // dP0^T, exp(S0)
      step(NK + ks);
      dpt[0] = mfma32(op[NK + ks], doreg[0][ks], dpt[0]);
      under_exp(0, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
    tail_exp(0);
    mask_block(0);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {           // S1^T, dS0
      step(2 * NK + ks);
      st[1] = mfma32(op[2 * NK + ks], qreg[0][ks], st[1]);
      under_ds(0, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
    tail_ds(0);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {           // dP1^T, exp(S1)
      step(3 * NK + ks);
      dpt[1] = mfma32(op[3 * NK + ks], doreg[0][ks], dpt[1]);
      under_exp(1, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
    tail_exp(1);
    mask_block(1);
#pragma unroll
    for (int m = 0; m < NK; ++m) {              // dQ0^T, dS1
      step(4 * NK + m);
      acc[0][m >> 1] = mfma32(op[4 * NK + m], dsb[0][m & 1], acc[0][m >> 1]);
      under_ds(1, m);
      __builtin_amdgcn_sched_barrier(0);
    }
    tail_ds(1);
#pragma unroll
    for (int m = 0; m < NK; ++m) {              // dQ1^T
      step(5 * NK + m);
      acc[0][m >> 1] = mfma32(op[5 * NK + m], dsb[1][m & 1], acc[0][m >> 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, std::integral_constant<int, 0>{});
    if (j + 1 < ntiles) tile(j + 1, std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (!row_ok[qb]) continue;
    const int r = wave * QW + qb * 32 + col;
    float* dst = a.dq + ((int64_t)(it.row0 + r) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4* p = (f32x4*)(dst + db * 32 + 8 * i4 + 4 * hh);
        f32x4 v = *p;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += a.scale * acc[qb][db][4 * i4 + e];
        *p = v;
      }
  }
}

// ---------------------------------------------------------------------------
// dkv kernel (bf16)
// ---------------------------------------------------------------------------
template <int D, int NW>
__device__ __forceinline__ void bwd_dkv_body(const BwdArgs& a, int bid, uint16_t* smem) {
  constexpr int BQ = kBwdBQ;                 // query rows per LDS tile (one 32-row MFMA block)
  constexpr int BK = 32 * NW;                // keys per workgroup
  uint16_t* s_v = smem;                                                   // [BK][D], loaded once
  uint16_t (*s_q)[BQ * D] = (uint16_t (*)[BQ * D])(smem + BK * D);       // [2][BQ][D]
  uint16_t (*s_do)[BQ * D] = (uint16_t (*)[BQ * D])(smem + BK * D + 2 * BQ * D);
  float (*s_lse)[64] = (float (*)[64])(smem + BK * D + 4 * BQ * D);      // [2][64]
  float (*s_dl)[64] = (float (*)[64])(smem + BK * D + 4 * BQ * D + 256);

  int item_rank, hdummy, g;
  map_block(bid, 1, a.hkv, item_rank, hdummy, g);
  if (item_rank >= a.hdr_k->n_items) return;
  const WorkItem it = a.items_k[a.order_k[item_rank]];
  if (it.nseg == 0) return;

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col = lane & 31, hh = lane >> 5;
  const int kr_ = wave * 32 + col;                  // key row in the tile
  const bool key_ok = kr_ < it.nrows;
  const KeyRanges qrng = query_ranges(a.mask, it.pos0 + kr_, a.tf_b, a.tf_n);

  // V rows of the whole key tile go to LDS once (B operand of dP = dO V^T
  // is read from there); K stays in registers as the B operand of S = Q K^T:
  // lane holds K[key][16*ks + 8*hh + 0..7].
  {
    TileLoader<D, BK, NW> lvv;
    const int64_t vst = a.v_st * 2;
    lvv.init(vst, wave, lane);
    lvv.issue(s_v, (const char*)a.v + ((int64_t)g * a.v_sh + (int64_t)it.row0 * a.v_st) * 2, it.nrows, vst);
  }
  bf16x8 kreg[D / 16];
  {
    const uint16_t* ks_ = (const uint16_t*)a.k + (int64_t)(it.row0 + kr_) * a.k_st + (int64_t)g * a.k_sh + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 rk = {0u, 0u, 0u, 0u};
      if (key_ok) rk = *(const u32x4*)(ks_ + 16 * ks);
      kreg[ks] = __builtin_bit_cast(bf16x8, rk);
    }
  }

  const int64_t qst = a.q_st * 2, dst_ = a.do_st * 2;
  TileLoader<D, BQ, NW> lq, ld;
  lq.init(qst, wave, lane);
  ld.init(dst_, wave, lane);
  const int nt0 = ceil_div(it.seg[0].n, BQ);
  const int nt1 = it.nseg > 1 ? ceil_div(it.seg[1].n, BQ) : 0;
  const int ntiles = (nt0 + nt1) * a.grp;
  // Query tiles run from the last segment's top tile downwards, and the
  // q-heads of the GQA group innermost.  Every key tile of a sequence's
  // chunk pair then starts on the same query rows and sweeps them in the
  // same order, each stopping at its own diagonal, so the workgroups that
  // run side by side on one XCD read each Q/dO tile from L2 at about the
  // same time instead of each fetching its own rows.  The position
  // advances without division; segment fields are picked by select so they
  // stay in scalar registers.
  struct TilePos { int h, s, t0; };
  auto seg_n = [&](int sgi) { return sgi ? it.seg[1].n : it.seg[0].n; };
  const int h_lo = g * a.grp, h_hi = h_lo + a.grp;
  auto next_pos = [&](TilePos tp) {
    ++tp.h;
    if (tp.h >= h_hi) {
      tp.h = h_lo;
      tp.t0 -= BQ;
      if (tp.t0 < 0) {   // down to segment 0 (only reached from segment 1)
        tp.s = 0;
        tp.t0 = (nt0 - 1) * BQ;
      }
    }
    return tp;
  };
  auto issue = [&](const TilePos& tp, int buf) {
    const int nvalid = min(BQ, seg_n(tp.s) - tp.t0);
    const int64_t row = (tp.s ? it.seg[1].row : it.seg[0].row) + tp.t0;
    lq.issue(s_q[buf], (const char*)a.q + (row * a.q_st + (int64_t)tp.h * a.q_sh) * 2, nvalid, qst);
    ld.issue(s_do[buf], (const char*)a.dout + (row * a.do_st + (int64_t)tp.h * a.do_sh) * 2, nvalid, dst_);
    if (wave < 2) {
      // LSE (wave 0) or delta (wave 1) of the tile's rows; rows past the
      // segment read as 0 and are masked
      const float* src = (wave == 0 ? a.lse : a.delta) + (int64_t)tp.h * a.tq + row;
      float* dstl = wave == 0 ? s_lse[buf] : s_dl[buf];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(src, (unsigned)(nvalid * 4)),
                                               (__attribute__((address_space(3))) void*)dstl, 4, lane * 4, 0, 0, 0);
    }
  };
  TilePos cur = nt1 > 0 ? TilePos{h_lo, 1, (nt1 - 1) * BQ} : TilePos{h_lo, 0, (nt0 - 1) * BQ};  // tile computed
  TilePos nxt = next_pos(cur);      // tile loaded next
  issue(cur, 0);

  f32x16 acc_k[D / 32], acc_v[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc_k[db][i] = 0.f; acc_v[db][i] = 0.f; }

  constexpr int NK = D / 16;     // k-steps of S and dP
  constexpr int NT = D / 8;      // dV and dK products
  constexpr int PF = kDkvPF, TPF = kDkvTPF;
  auto tile = [&](int j, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_loads();
    __syncthreads();
    if (j + 1 < ntiles) issue(nxt, buf ^ 1);
    const int t0 = cur.t0;
    const int sn = seg_n(cur.s);
    const int spos = cur.s ? it.seg[1].pos : it.seg[0].pos;
    const bool full = t0 >= (cur.s ? it.seg[1].full_lo : it.seg[0].full_lo) &&
                      t0 + BQ <= (cur.s ? it.seg[1].full_hi : it.seg[0].full_hi);
    cur = nxt;
    nxt = next_pos(nxt);
    const uint16_t* tq = s_q[buf];
    const uint16_t* tdo = s_do[buf];

    // The tile is software-pipelined by hand: operand reads are issued PF
    // (S, dP) or TPF (dV, dK) products ahead, and each step is fenced so
    // the order stays as written. Per wave: S = Q K^T (one accumulator
    // chain), then dP = dO V^T with P = exp(S*scale - lse) computed under
    // it, then dV^T += dO^T P^T with dS = P * (dP - delta) computed under
    // it, then dK^T += Q^T dS^T. Accumulator element i of a lane holds
    // query row 8*(i/4) + 4*hh + i%4 and key column `col`.
    f32x16 st, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) { st[i] = 0.f; dp[i] = 0.f; }
    bf16x8 qa[NK], da[NK], va[NK];
    auto read_sdp = [&](int u) {  // operands of product u of the S, dP sequence
      if (u < NK) {
        qa[u] = read_row8<D>(tq, 0, col, u, hh);
      } else {
        da[u - NK] = read_row8<D>(tdo, 0, col, u - NK, hh);
        va[u - NK] = read_row8<D>(s_v, wave * 32, col, u - NK, hh);
      }
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) read_sdp(u);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      if (ks + PF < 2 * NK) read_sdp(ks + PF);
      st = mfma32(qa[ks], kreg[ks], st);
      __builtin_amdgcn_sched_barrier(0);
    }
    // exp of the 4 rows of group g4 (lse read two products earlier); a row
    // with lse = -inf has no allowed key: it only occurs in partial tiles,
    // where the mask below zeroes it
    f32x4 l4[4];
    auto exp_group = [&](int g4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = __builtin_amdgcn_exp2f(st[4 * g4 + e] * a.scale_log2 - l4[g4][e] * 1.4426950408889634f);
        asm("" : "+v"(pv));  // opaque to folds: the exp stays ahead of the mask branch
        st[4 * g4 + e] = pv;
      }
    };
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      if (NK + ks + PF < 2 * NK) read_sdp(NK + ks + PF);
      if (ks < 4) l4[ks] = *(const f32x4*)(&s_lse[buf][4 * hh + 8 * ks]);
      dp = mfma32(da[ks], va[ks], dp);
      if (ks >= 2 && ks < 6) exp_group(ks - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g4 = NK - 2; g4 < 4; ++g4) exp_group(g4);  // groups past the last product (D = 64)

    bf16x8 ta[NT];
    auto read_t = [&](int m) {  // operand of product m: dV (m < NT/2) or dK
      const int hf = (m % (NT / 2)) / (D / 32), db = m % (D / 32);
      ta[m] = read_tr<D>(m < NT / 2 ? tdo : tq, 16 * hf, 32 * db, lane);
    };
#pragma unroll
    for (int m = 0; m < TPF; ++m) read_t(m);
    if (!full) {
      const int qofs0 = t0 + 4 * hh;
      const int rem = sn - qofs0;
      const int pbase = spos + qofs0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 8 * (i >> 2) + (i & 3);
        st[i] = ((off < rem) & in_ranges(qrng, pbase + off)) ? st[i] : 0.f;
      }
    }
    const bf16x8 pb[2] = {pack_b(st, 0), pack_b(st, 1)};
    bf16x8 ds[2];
    f32x4 d4[4];
    auto ds_group = [&](int g4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * g4 + e] = st[4 * g4 + e] * (dp[4 * g4 + e] - d4[g4][e]);
    };
#pragma unroll
    for (int m = 0; m < NT / 2; ++m) {
      if (m + TPF < NT) read_t(m + TPF);
      if (m < 4) d4[m] = *(const f32x4*)(&s_dl[buf][4 * hh + 8 * m]);
      const int hf = m / (D / 32), db = m % (D / 32);
      acc_v[db] = mfma32(ta[m], pb[hf], acc_v[db]);
      if (m >= 1 && m <= 4) ds_group(m - 1);
      if (m == 3) ds[0] = pack_b(dp, 0);
      if (m == 5) ds[1] = pack_b(dp, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // groups and packs past the last dV product (D = 64)
#pragma unroll
    for (int g4 = NT / 2 - 1; g4 < 4; ++g4) ds_group(g4);
    if (3 >= NT / 2) ds[0] = pack_b(dp, 0);
    if (5 >= NT / 2) ds[1] = pack_b(dp, 1);
#pragma unroll
    for (int m = NT / 2; m < NT; ++m) {
      if (m + TPF < NT) read_t(m + TPF);
      const int hf = (m - NT / 2) / (D / 32), db = m % (D / 32);
      acc_k[db] = mfma32(ta[m], ds[hf], acc_k[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, std::integral_constant<int, 0>{});
    if (j + 1 < ntiles) tile(j + 1, std::integral_constant<int, 1>{});
  }

  if (!key_ok) return;
  const int64_t row = it.row0 + kr_;
  float* dkp = a.dk + (row * a.hkv + g) * D;
  float* dvp = a.dv + (row * a.hkv + g) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int off = db * 32 + 8 * i4 + 4 * hh;
      f32x4 vk = *(f32x4*)(dkp + off), vv = *(f32x4*)(dvp + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vk[e] += a.scale * acc_k[db][4 * i4 + e];
        vv[e] += acc_v[db][4 * i4 + e];
      }
      *(f32x4*)(dkp + off) = vk;
      *(f32x4*)(dvp + off) = vv;
    }
}

// One launch per step: workgroups [0, dkv_blocks) take key tiles (the longer
// items, dispatched first), the rest take query tiles.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_bf16_kernel(BwdArgs a) {
  constexpr int DQ_LDS = 4 * kBwdBK * D;                            // 2 x (K, V) tiles
  constexpr int DKV_LDS = 32 * kDkvWaves * D + 4 * kBwdBQ * D + 512; // V tile + 2 x (Q, dO) + lse, delta
  constexpr int LDS = DQ_LDS > DKV_LDS ? DQ_LDS : DKV_LDS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[LDS];
  static_assert(kDqWaves == 4 && kDkvWaves == 4, "both bodies run 256 threads");
  const int bid = blockIdx.x;
  if (bid < a.dkv_blocks) bwd_dkv_body<D, kDkvWaves>(a, bid, smem);
  else bwd_dq_body<D, kDqWaves, kDqQB>(a, bid - a.dkv_blocks, smem);
}

// ---------------------------------------------------------------------------
// fp32 path: one row per thread.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(BwdArgs a) {
  int item_rank, h, g;
  map_block(blockIdx.x, a.grp, a.hkv, item_rank, h, g);
  if (item_rank >= a.hdr_q->n_items) return;
  const WorkItem it = a.items_q[a.order_q[item_rank]];
  const int r = threadIdx.x;
  if (r >= it.nrows) return;
  const int64_t row = it.row0 + r;
  const int pq = it.pos0 + r;
  const float* qp = (const float*)a.q + row * a.q_st + (int64_t)h * a.q_sh;
  const float* dop = (const float*)a.dout + row * a.do_st + (int64_t)h * a.do_sh;
  const float l = a.lse[(int64_t)h * a.tq + row];
  if (l == -INFINITY) return;
  const float dl = a.delta[(int64_t)h * a.tq + row];
  float qv[D], dov[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { qv[c] = qp[c]; dov[c] = dop[c]; acc[c] = 0.f; }
  for (int s = 0; s < it.nseg; ++s) {
    const Segment sg = it.seg[s];
    for (int kk = 0; kk < sg.n; ++kk) {
      if (!mask_allowed(a.mask, pq, sg.pos + kk, a.tf_b, a.tf_n)) continue;
      const float* kr = (const float*)a.k + (int64_t)(sg.row + kk) * a.k_st + (int64_t)g * a.k_sh;
      const float* vr = (const float*)a.v + (int64_t)(sg.row + kk) * a.v_st + (int64_t)g * a.v_sh;
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) { sdot = fmaf(qv[c], kr[c], sdot); pdot = fmaf(dov[c], vr[c], pdot); }
      const float p = expf(sdot * a.scale - l);
      const float ds = p * (pdot - dl);
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, kr[c], acc[c]);
    }
  }
  float* dst = a.dq + (row * a.hq + h) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) dst[c] += a.scale * acc[c];
}

template <int D>
__global__ __launch_bounds__(64) void bwd_dkv_f32_kernel(BwdArgs a) {
  int item_rank, hdummy, g;
  map_block(blockIdx.x, 1, a.hkv, item_rank, hdummy, g);
  if (item_rank >= a.hdr_k->n_items) return;
  const WorkItem it = a.items_k[a.order_k[item_rank]];
  const int r = threadIdx.x;
  if (r >= it.nrows) return;
  const int64_t row = it.row0 + r;
  const int pk = it.pos0 + r;
  const float* kp = (const float*)a.k + row * a.k_st + (int64_t)g * a.k_sh;
  const float* vp = (const float*)a.v + row * a.v_st + (int64_t)g * a.v_sh;
  float kv[D], vv[D], ak[D], av[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { kv[c] = kp[c]; vv[c] = vp[c]; ak[c] = 0.f; av[c] = 0.f; }
  for (int jh = 0; jh < a.grp; ++jh) {
    const int h = g * a.grp + jh;
    for (int s = 0; s < it.nseg; ++s) {
      const Segment sg = it.seg[s];
      for (int qq = 0; qq < sg.n; ++qq) {
        if (!mask_allowed(a.mask, sg.pos + qq, pk, a.tf_b, a.tf_n)) continue;
        const int64_t qrow = sg.row + qq;
        const float l = a.lse[(int64_t)h * a.tq + qrow];
        if (l == -INFINITY) continue;
        const float* qr = (const float*)a.q + qrow * a.q_st + (int64_t)h * a.q_sh;
        const float* dr = (const float*)a.dout + qrow * a.do_st + (int64_t)h * a.do_sh;
        float sdot = 0.f, pdot = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) { sdot = fmaf(qr[c], kv[c], sdot); pdot = fmaf(dr[c], vv[c], pdot); }
        const float p = expf(sdot * a.scale - l);
        const float ds = p * (pdot - a.delta[(int64_t)h * a.tq + qrow]);
#pragma unroll
        for (int c = 0; c < D; ++c) { ak[c] = fmaf(ds, qr[c], ak[c]); av[c] = fmaf(p, dr[c], av[c]); }
      }
    }
  }
  float* dkp = a.dk + (row * a.hkv + g) * D;
  float* dvp = a.dv + (row * a.hkv + g) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) { dkp[c] += a.scale * ak[c]; dvp[c] += av[c]; }
}

}  // namespace

int bwd_dq_tile_rows(bool bf16) { return bf16 ? 32 * kDqQB * kDqWaves : 64; }
int bwd_dkv_tile_rows(bool bf16) { return bf16 ? 32 * kDkvWaves : 64; }

hipError_t launch_bwd(BwdArgs a, bool bf16, int d, int64_t max_items_q, int64_t max_items_k, hipStream_t stream) {
  const unsigned gq = unit_grid(max_items_q, a.hkv, a.grp);
  const unsigned gk = unit_grid(max_items_k, a.hkv, 1);
  if (bf16) {
    a.dkv_blocks = (int)gk;
    const dim3 grid(gk + unit_grid(max_items_q, a.hkv, a.grp, items_per_unit(a.grp)));
    if (d == 128) hipLaunchKernelGGL(bwd_bf16_kernel<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(bwd_bf16_kernel<64>, grid, dim3(256), 0, stream, a);
  } else {
    a.dkv_blocks = 0;
    if (d == 128) {
      hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, dim3(gq), dim3(64), 0, stream, a);
      hipLaunchKernelGGL(bwd_dkv_f32_kernel<128>, dim3(gk), dim3(64), 0, stream, a);
    } else {
      hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3(gq), dim3(64), 0, stream, a);
      hipLaunchKernelGGL(bwd_dkv_f32_kernel<64>, dim3(gk), dim3(64), 0, stream, a);
    }
  }
  return hipGetLastError();
}

}  // namespace cpattn
