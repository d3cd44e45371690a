// Varlen tile scheduler (device prologue).
//
// Packed sequences arrive as THD tensors with cu_seqlens ("Speeding up
// Variable-Length Training with Dynamic Context Parallelism and NVIDIA
// Megatron Core", section A2), and attention work per sequence grows with
// the square of its length (same page, data scheduling model), so a flat
// grid over tokens leaves most of the chip idle behind one long sequence.
// This kernel turns (cu_seqlens, ring step, mask) into a work list:
//   * one item per primary tile (query tile for the forward and dQ passes,
//     key tile for the dK/dV pass) inside one zigzag chunk of one sequence;
//   * per item up to two segments on the other side holding every row the
//     tile can interact with under the mask; tiles with no allowed pair are
//     never visited, and rows allowed for the whole tile are marked so the
//     attention kernels skip the element mask there;
//   * items sorted by cost, longest first, so long sequences start early.
// Each schedule is one 1024-thread workgroup (the backward builds its two
// lists in one launch, one workgroup each); it also validates the device
// cu_seqlens arrays (a bad array yields zero items and an error status).
#include "common.h"

namespace cpattn {

namespace {

constexpr int kThreads = 1024;
constexpr int kBins = 2048;
// Per-sequence item offsets and per-item costs also stay in LDS when they
// fit, so the binary search and the final scatter do not wait on global
// memory written moments before; larger batches read them from the workspace.
constexpr int kLdsSeqs = 2048;
constexpr int kLdsItems = 8192;

__device__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      int t = s_wave[w];
      s_wave[w] = acc;
      acc += t;
    }
    s_wave[kThreads / 64] = acc;
  }
  __syncthreads();
  int res = s_wave[wave] + incl - v;
  *total = s_wave[kThreads / 64];
  __syncthreads();
  return res;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ void set_seg(Segment& s, int row_base, int pos_base, int lo, int hi, int flo, int fhi) {
  s.row = row_base + lo;
  s.pos = pos_base + lo;
  s.n = hi - lo;
  flo = clampi(flo, lo, hi);
  fhi = clampi(fhi, lo, hi);
  if (fhi <= flo) { flo = 0; fhi = 0; } else { flo -= lo; fhi -= lo; }
  s.full_lo = flo;
  s.full_hi = fhi;
}

// Clean-stream key extent of a teacher-forcing query at position p:
// keys [0, E) of the clean stream are allowed (chunks <= c for clean
// queries, chunks < c for noisy ones).
__device__ __forceinline__ int tf_clean_extent(int p, int B, int span) {
  return p < span ? (p / B + 1) * B : ((p - span) / B) * B;
}

// Segments of secondary rows for a primary tile with positions [p0, p1).
// Secondary chunk list: (row_base, pos_base, len) for up to 2 chunks.
__device__ int build_segments(const SchedArgs& a, int p0, int p1, const int* cb, const int* cpos,
                              const int* clen, int nchunks, Segment* seg) {
  int ns = 0;
  if (a.mask == CPATTN_MASK_BIDIR) {
    for (int c = 0; c < nchunks; ++c)
      if (clen[c] > 0) set_seg(seg[ns++], cb[c], cpos[c], 0, clen[c], 0, clen[c]);
    return ns;
  }
  if (a.mask == CPATTN_MASK_CAUSAL) {
    for (int c = 0; c < nchunks; ++c) {
      const int A = cpos[c], C = clen[c];
      if (C <= 0) continue;
      if (a.primary_is_q) {
        // keys with position <= p1-1; allowed for all rows: position <= p0
        const int hi = clampi(p1 - A, 0, C);
        if (hi > 0) set_seg(seg[ns++], cb[c], A, 0, hi, 0, clampi(p0 + 1 - A, 0, C));
      } else {
        // queries with position >= p0; allowed for all keys: >= p1-1
        const int lo = clampi(p0 - A, 0, C);
        if (lo < C) set_seg(seg[ns++], cb[c], A, lo, C, clampi(p1 - 1 - A, 0, C), C);
      }
    }
    return ns;
  }
  // Teacher forcing at cp = 1 (a single chunk holding the whole sequence);
  // cp > 1 uses the balanced split (build_item_tf).
  const int B = a.tf_b, span = a.tf_b * a.tf_n, L = 2 * span;
  const int base = cb[0];
  const bool has_clean = p0 < span, has_noisy = p1 > span;
  if (a.primary_is_q) {
    int hi = 0, full = 1 << 30;
    if (has_clean) {
      hi = max(hi, tf_clean_extent(min(p1, span) - 1, B, span));
      full = min(full, tf_clean_extent(p0, B, span));
    }
    if (has_noisy) {
      hi = max(hi, tf_clean_extent(p1 - 1, B, span));
      full = min(full, tf_clean_extent(max(p0, span), B, span));
    }
    if (hi > 0) set_seg(seg[ns++], base, 0, 0, hi, 0, min(full, hi));
    if (has_noisy) {
      const int clo = (max(p0, span) - span) / B, chi = (p1 - 1 - span) / B;
      const int lo = span + clo * B, h2 = span + (chi + 1) * B;
      const bool full_all = !has_clean && clo == chi;
      set_seg(seg[ns++], base, 0, lo, h2, full_all ? lo : 0, full_all ? h2 : 0);
    }
    return ns;
  }
  // primary = keys [p0, p1)
  if (has_clean && has_noisy) {
    // the tile straddles the stream boundary: its noisy keys are chunks
    // 0..nk_hi.  Clean queries of chunks >= ck_lo and noisy queries of
    // chunks <= nk_hi form one run [ck_lo*B, span + (nk_hi+1)*B); noisy
    // queries of chunks > ck_lo (which see the clean keys) add the suffix
    // past it.  Every row of both runs attends some key of the tile.
    const int ck_lo = p0 / B, nk_hi = (p1 - 1 - span) / B;
    const int run_hi = span + (nk_hi + 1) * B, suf_lo = span + (ck_lo + 1) * B;
    if (suf_lo <= run_hi) {
      set_seg(seg[ns++], base, 0, ck_lo * B, max(run_hi, suf_lo < L ? L : run_hi), 0, 0);
    } else {
      set_seg(seg[ns++], base, 0, ck_lo * B, run_hi, 0, 0);
      if (suf_lo < L) set_seg(seg[ns++], base, 0, suf_lo, L, 0, 0);
    }
  } else if (has_clean) {
    const int ck_lo = p0 / B, ck_hi = (p1 - 1) / B;
    // clean queries of chunks >= ck_lo (all keys for chunks >= ck_hi)
    set_seg(seg[ns++], base, 0, ck_lo * B, span, ck_hi * B, span);
    // noisy queries of chunks > ck_lo (all keys for chunks > ck_hi)
    const int lo = span + (ck_lo + 1) * B;
    if (lo < L) set_seg(seg[ns++], base, 0, lo, L, span + (ck_hi + 1) * B, L);
  } else {
    const int nk_lo = (p0 - span) / B, nk_hi = (p1 - 1 - span) / B;
    const int lo = span + nk_lo * B, hi = span + (nk_hi + 1) * B;
    const bool full_all = nk_lo == nk_hi;
    set_seg(seg[ns++], base, 0, lo, hi, full_all ? lo : 0, full_all ? hi : 0);
  }
  return ns;
}

// Balanced teacher-forcing split at cp > 1 ("Scaling Video Training with
// Parallelism", section 4, balanced SP): time chunks are dealt to ranks in
// snake order over rounds of 2cp (tf_owner), and a rank's local rows are its
// m = N/cp clean chunks in ascending order, then its noisy chunks in the same
// order, B rows each.  Primary tiles never straddle a chunk block, and under
// the teacher-forcing mask a block either sees another block completely or
// not at all, so every segment below is fully allowed and the attention
// kernels run it unmasked (only rows past a segment end are cut).  In local
// block indices of the secondary rank rs:
//   clean query of chunk c   clean blocks of chunks <= c        (a prefix)
//   noisy query of chunk c   clean blocks of chunks < c         (a prefix)
//                            + noisy block of chunk c if rs holds it
//   clean key of chunk c     clean blocks of chunks >= c        (a suffix)
//                            + noisy blocks of chunks > c       (a suffix)
//   noisy key of chunk c     noisy block of chunk c if rs holds it
__device__ void build_item_tf(const SchedArgs& a, int pr0, int sr0, int t_in_seq, WorkItem& it) {
  const int cp = a.cp, B = a.tf_b, m = a.tf_n / cp, span = a.tf_b * a.tf_n;
  const int tpb = ceil_div(B, a.tile_p);
  const int blk = t_in_seq / tpb, t = t_in_seq - blk * tpb;
  const bool pn = blk >= m;                                      // primary block is noisy
  const int pc = tf_rank_chunk(a.rank_p, pn ? blk - m : blk, cp);  // its time chunk
  it.row0 = pr0 + blk * B + t * a.tile_p;
  it.nrows = min(a.tile_p, B - t * a.tile_p);
  it.pos0 = (pn ? span : 0) + pc * B + t * a.tile_p;
  const int rs = a.rank_s;
  int ns = 0;
  auto seg = [&](int lo, int hi) {    // local blocks [lo, hi) of rank rs
    const int first = lo < m ? tf_rank_chunk(rs, lo, cp) * B : span + tf_rank_chunk(rs, lo - m, cp) * B;
    Segment& g = it.seg[ns++];
    g.row = sr0 + lo * B;
    g.pos = first;
    g.n = (hi - lo) * B;
    g.full_lo = 0;
    g.full_hi = g.n;
  };
  const int below = tf_count_below(rs, pc, cp);       // rs's chunks < pc
  const int upto = tf_count_below(rs, pc + 1, cp);    // rs's chunks <= pc
  const bool holds = tf_owner(pc, cp) == rs;
  if (a.primary_is_q) {
    if (!pn) {
      if (upto > 0) seg(0, upto);
    } else {
      if (below > 0) seg(0, below);
      if (holds) seg(m + below, m + below + 1);
    }
  } else if (!pn) {
    if (below < m) seg(below, m);
    if (upto < m) seg(m + upto, 2 * m);
  } else if (holds) {
    seg(m + below, m + below + 1);
  }
  it.nseg = ns;
}

__device__ __forceinline__ void sched_body(const SchedArgs& a) {
  __shared__ int s_err;
  __shared__ int s_wave[kThreads / 64 + 1];
  __shared__ int s_bins[kBins];
  __shared__ int s_seq_base[kLdsSeqs + 1];
  __shared__ int s_cu_p[kLdsSeqs + 1], s_cu_s[kLdsSeqs + 1];
  __shared__ unsigned short s_bin_of[kLdsItems];
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0;
  for (int i = tid; i < kBins; i += kThreads) s_bins[i] = 0;
  __syncthreads();

  const int cp = a.cp;
  // ---- pass 1: validate, count tiles per sequence, prefix sum -------------
  int carry = 0;
  for (int b0 = 0; b0 < a.nseq; b0 += kThreads) {
    const int b = b0 + tid;
    int cnt = 0;
    if (b < a.nseq) {
      const int p0 = a.cu_p[b], p1 = a.cu_p[b + 1];
      const int s0 = a.cu_s[b], s1 = a.cu_s[b + 1];
      if (a.nseq <= kLdsSeqs) {
        s_cu_p[b + 1] = p1;
        s_cu_s[b + 1] = s1;
        if (b == 0) {
          s_cu_p[0] = p0;
          s_cu_s[0] = s0;
        }
      }
      bool bad = (b == 0 && (p0 != 0 || s0 != 0)) || p1 < p0 || s1 < s0 ||
                 (int64_t)p1 > a.tokens_p || (int64_t)s1 > a.tokens_s;
      const int lp = p1 - p0, ls = s1 - s0;
      const bool tfs = a.mask == CPATTN_MASK_TF_BLOCK && cp > 1;   // balanced teacher-forcing split
      // zigzag halves matter only where positions do; BIDIR takes any split
      const bool halves = cp > 1 && a.mask != CPATTN_MASK_BIDIR;
      if (cp > 1) bad = bad || (halves && (lp & 1)) || lp != ls;
      if (a.mask == CPATTN_MASK_TF_BLOCK) bad = bad || lp != ls || lp != 2 * a.tf_b * (a.tf_n / cp);
      if (bad) atomicOr(&s_err, 1);
      if (!bad) {
        if (tfs) cnt = 2 * (a.tf_n / cp) * ceil_div(a.tf_b, a.tile_p);
        else if (halves) cnt = 2 * ceil_div(lp >> 1, a.tile_p);
        else cnt = ceil_div(lp, a.tile_p);
      }
    }
    int tot;
    const int ex = block_excl_scan(cnt, s_wave, &tot);
    if (b < a.nseq) {
      a.seq_base[b] = carry + ex;
      if (a.nseq <= kLdsSeqs) s_seq_base[b] = carry + ex;
    }
    carry += tot;
  }
  // rows past the last sequence (a padded buffer): items without segments,
  // so the forward still writes every row (0 and lse = -inf)
  __shared__ int s_tail;
  if (tid == 0) {
    a.seq_base[a.nseq] = carry;
    if (a.nseq <= kLdsSeqs) s_seq_base[a.nseq] = carry;
    const int64_t end = a.nseq > 0 ? (int64_t)a.cu_p[a.nseq] : 0;
    const int64_t rest = a.tail_items && end < a.tokens_p ? a.tokens_p - end : 0;
    s_tail = (int)((rest + a.tile_p - 1) / a.tile_p);
    if ((int64_t)carry + s_tail > a.max_items) s_err = 1;
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) {
      a.hdr->status = CPATTN_ERR_INVALID_ARG;
      a.hdr->n_items = 0;
    }
    return;
  }
  const int n_seq_items = carry;
  const int n_items = carry + s_tail;

  // ---- pass 2: build items -------------------------------------------------
  for (int idx = tid; idx < n_items; idx += kThreads) {
    if (idx >= n_seq_items) {
      const int end = a.nseq > 0 ? a.cu_p[a.nseq] : 0;
      WorkItem it;
      it.seq = a.nseq;
      it.row0 = end + (idx - n_seq_items) * a.tile_p;
      it.nrows = (int)min((int64_t)a.tile_p, a.tokens_p - it.row0);
      it.pos0 = 0;
      it.cost = 0;
      it.nseg = 0;
      it.seg[0] = Segment{0, 0, 0, 0, 0};
      it.seg[1] = Segment{0, 0, 0, 0, 0};
      a.items[idx] = it;
      atomicAdd(&s_bins[0], 1);
      if (idx < kLdsItems) s_bin_of[idx] = 0;
      continue;
    }
    // sequence: last b with seq_base[b] <= idx
    const int* sb = a.nseq <= kLdsSeqs ? s_seq_base : a.seq_base;
    int lo = 0, hi = a.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sb[mid] <= idx) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int t_in_seq = idx - sb[b];
    const int* cup = a.nseq <= kLdsSeqs ? s_cu_p : a.cu_p;
    const int* cus = a.nseq <= kLdsSeqs ? s_cu_s : a.cu_s;
    const int pr0 = cup[b], lp = cup[b + 1] - pr0;
    const int sr0 = cus[b], ls = cus[b + 1] - sr0;
    if (a.mask == CPATTN_MASK_TF_BLOCK && cp > 1) {
      WorkItem it;
      it.seq = b;
      it.seg[0] = Segment{0, 0, 0, 0, 0};
      it.seg[1] = Segment{0, 0, 0, 0, 0};
      build_item_tf(a, pr0, sr0, t_in_seq, it);
      int cost = 0;
      for (int s = 0; s < it.nseg; ++s) cost += ceil_div(it.seg[s].n, a.tile_s);
      it.cost = cost * a.cost_mult;
      a.items[idx] = it;
      atomicAdd(&s_bins[min(it.cost, kBins - 1)], 1);
      if (idx < kLdsItems) s_bin_of[idx] = (unsigned short)min(it.cost, kBins - 1);
      continue;
    }
    const bool halves = cp > 1 && a.mask != CPATTN_MASK_BIDIR;
    int chunk_off = 0, chunk_len = lp, t = t_in_seq;
    if (halves) {
      const int half = lp >> 1, per = ceil_div(half, a.tile_p);
      const int hsel = t_in_seq >= per ? 1 : 0;
      t = t_in_seq - hsel * per;
      chunk_off = hsel * half;
      chunk_len = half;
    }
    const int off0 = chunk_off + t * a.tile_p;
    const int nrows = min(a.tile_p, chunk_len - t * a.tile_p);
    WorkItem it;
    it.seq = b;
    it.row0 = pr0 + off0;
    it.nrows = nrows;
    it.pos0 = halves ? zigzag_pos(off0, lp, cp, a.rank_p) : off0;
    int cb[2], cpos[2], clen[2], nch;
    if (halves) {
      const int half = ls >> 1;
      nch = 2;
      cb[0] = sr0;        cpos[0] = a.rank_s * half;                clen[0] = half;
      cb[1] = sr0 + half; cpos[1] = (2 * cp - 1 - a.rank_s) * half; clen[1] = half;
    } else {
      nch = 1;
      cb[0] = sr0; cpos[0] = 0; clen[0] = ls;
    }
    it.seg[0] = Segment{0, 0, 0, 0, 0};
    it.seg[1] = Segment{0, 0, 0, 0, 0};
    it.nseg = build_segments(a, it.pos0, it.pos0 + nrows, cb, cpos, clen, nch, it.seg);
    int cost = 0;
    for (int s = 0; s < it.nseg; ++s) cost += ceil_div(it.seg[s].n, a.tile_s);
    it.cost = cost * a.cost_mult;
    a.items[idx] = it;
    atomicAdd(&s_bins[min(it.cost, kBins - 1)], 1);
    if (idx < kLdsItems) s_bin_of[idx] = (unsigned short)min(it.cost, kBins - 1);
  }
  __syncthreads();

  // ---- pass 3: bin offsets, highest cost first -----------------------------
  {
    // thread tid owns bins (kBins-1-2*tid) and (kBins-2-2*tid)
    const int bA = kBins - 1 - 2 * tid, bB = kBins - 2 - 2 * tid;
    const int cA = s_bins[bA], cB = s_bins[bB];
    int tot;
    const int ex = block_excl_scan(cA + cB, s_wave, &tot);
    s_bins[bA] = ex;
    s_bins[bB] = ex + cA;
  }
  __syncthreads();

  // ---- pass 4: scatter ---------------------------------------------------------
  for (int idx = tid; idx < n_items; idx += kThreads) {
    const int bin = idx < kLdsItems ? (int)s_bin_of[idx] : min(a.items[idx].cost, kBins - 1);
    const int pos = atomicAdd(&s_bins[bin], 1);
    a.order[pos] = idx;
  }
  if (tid == 0) {
    a.hdr->status = CPATTN_OK;
    a.hdr->n_items = n_items;
  }
}

__global__ __launch_bounds__(kThreads) void sched_kernel(SchedArgs a) { sched_body(a); }

// Two independent schedules (disjoint workspace regions) in one launch, one
// workgroup each: the backward's query-tile and key-tile lists.
__global__ __launch_bounds__(kThreads) void sched_pair_kernel(SchedArgs a, SchedArgs b) {
  if (blockIdx.x == 0) sched_body(a);
  else sched_body(b);
}

}  // namespace

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sched_pair(const SchedArgs& a, const SchedArgs& b, hipStream_t stream) {
  hipLaunchKernelGGL(sched_pair_kernel, dim3(2), dim3(kThreads), 0, stream, a, b);
  return hipGetLastError();
}

}  // namespace cpattn
