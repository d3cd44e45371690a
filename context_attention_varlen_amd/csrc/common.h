// Internal definitions shared by the libcpattn HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>
#include <stdint.h>

#include "cpattn.h"

namespace cpattn {

// ---------------------------------------------------------------------------
// Work items built by the device-side varlen tile scheduler.
//
// A work item is one tile of rows on the "primary" side (query rows for the
// forward and the dQ pass, key rows for the dK/dV pass) inside one zigzag
// chunk of one sequence, plus up to two segments of rows on the other side
// that hold every row the tile may attend (or be attended by).  Inside a
// segment, rows [full_lo, full_hi) are allowed for every primary row of the
// tile, so tiles lying inside that range need no element mask.
// ---------------------------------------------------------------------------
struct Segment {
  int32_t row;      // absolute tensor row of the segment's first row
  int32_t pos;      // in-sequence position of that row
  int32_t n;        // rows in the segment
  int32_t full_lo;  // [full_lo, full_hi): offsets allowed for every tile row
  int32_t full_hi;
};

struct WorkItem {
  int32_t seq;
  int32_t row0;     // absolute tensor row of the tile's first primary row
  int32_t nrows;    // primary rows in this tile
  int32_t pos0;     // in-sequence position of the first primary row
  int32_t cost;     // secondary tiles to visit (sum over segments)
  int32_t nseg;
  Segment seg[2];
};
static_assert(sizeof(WorkItem) == 64, "work item is one 64-byte record");

// Workspace header (first 256 bytes of the workspace).
struct WsHeader {
  int32_t status;     // cpattn_status left by the last scheduler run
  int32_t n_items;    // items produced
  int32_t pad[62];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

struct SchedArgs {
  const int32_t* cu_p;   // cu_seqlens of the primary side (local)
  const int32_t* cu_s;   // cu_seqlens of the secondary side (local)
  int32_t nseq;
  int64_t tokens_p;      // rows of the primary tensor
  int64_t tokens_s;      // rows of the secondary tensor
  int32_t cp;
  int32_t rank_p;        // rank owning the primary rows
  int32_t rank_s;        // rank owning the secondary rows
  int32_t primary_is_q;  // 1: primary = queries, 0: primary = keys
  int32_t mask;
  int32_t tf_b, tf_n;
  int32_t tile_p;        // primary tile rows
  int32_t tile_s;        // secondary tile rows (cost unit)
  int32_t cost_mult;     // cost multiplier (GQA group size for the dK/dV pass)
  int32_t tail_items;    // 1: rows [cu_p[nseq], tokens_p) get items with no segments
  int32_t max_items;
  WsHeader* hdr;
  WorkItem* items;
  int32_t* order;        // items sorted by cost, descending
  int32_t* seq_base;     // [nseq + 1] first item of every sequence
};

// Workspace carve-up shared by host code: two schedule regions (A: query
// tiles, used by the forward and the dQ pass; B: key tiles, used by the
// dK/dV pass), each with a header, items, sorted order and per-sequence base.
struct WsRegion {
  size_t hdr, items, order, seq_base, end;
};
struct WsLayout {
  WsRegion a, b;
  size_t total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMinTile = 64;   // smallest primary tile any kernel uses

inline int64_t max_items_for(int64_t tokens, int32_t nseq, int tile) {
  // every sequence contributes at most two chunks, each with a ragged tail
  return (tokens + tile - 1) / tile + 2 * (int64_t)nseq + 1;
}

// Items one schedule region can hold: the zigzag bound at the smallest tile,
// plus room for the balanced teacher-forcing split, whose 2N/cp chunk blocks
// per sequence (at least 32 rows each) have a ragged tail each:
// T/tile + T/B <= T/64 + T/32 < T/16.
inline int64_t ws_item_capacity(int64_t tokens, int32_t nseq) {
  return (tokens + 15) / 16 + 2 * (int64_t)nseq + 1;
}

// Balanced teacher-forcing split (see the scheduler): time chunk c belongs to
// rank u or 2cp-1-u of its round, u = c mod 2cp; rank r's k-th chunk in
// ascending order; and how many of rank r's chunks lie below chunk c.
__host__ __device__ inline int32_t tf_owner(int32_t c, int32_t cp) {
  const int32_t u = c % (2 * cp);
  return u < cp ? u : 2 * cp - 1 - u;
}
__host__ __device__ inline int32_t tf_rank_chunk(int32_t r, int32_t k, int32_t cp) {
  return (k >> 1) * 2 * cp + ((k & 1) ? 2 * cp - 1 - r : r);
}
__host__ __device__ inline int32_t tf_count_below(int32_t r, int32_t c, int32_t cp) {
  const int32_t u = c % (2 * cp);
  return 2 * (c / (2 * cp)) + (r < u ? 1 : 0) + (2 * cp - 1 - r < u ? 1 : 0);
}

inline WsRegion ws_region(size_t base, int64_t tokens, int32_t nseq) {
  const int64_t mi = ws_item_capacity(tokens, nseq);
  WsRegion r;
  r.hdr = base;
  r.items = base + 256;
  r.order = align_up(r.items + mi * sizeof(WorkItem), 256);
  r.seq_base = align_up(r.order + mi * sizeof(int32_t), 256);
  r.end = align_up(r.seq_base + (nseq + 1) * sizeof(int32_t), 256);
  return r;
}

inline WsLayout ws_layout(int64_t tokens_q, int64_t tokens_k, int32_t nseq) {
  WsLayout L;
  L.a = ws_region(0, tokens_q, nseq);
  L.b = ws_region(L.a.end, tokens_k, nseq);
  L.total = L.b.end;
  return L;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  void* out;
  int64_t o_st, o_sh;
  float* lse;
  int64_t tq;          // lse row stride (query tokens)
  int hq, hkv, grp;
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  int mask, tf_b, tf_n;
  const WsHeader* hdr;
  const WorkItem* items;
  const int32_t* order;
  int order_cap;       // entries the order array holds (the scheduler's item bound)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, do_st, do_sh;
  const float* lse;     // [Hq][Tq]
  const float* delta;   // [Hq][Tq]
  int64_t tq;
  float* dq;            // [Tq][Hq][D] +=
  float* dk;            // [Tk][Hkv][D] +=
  float* dv;
  int hq, hkv, grp;
  float scale, scale_log2;
  int mask, tf_b, tf_n;
  const WsHeader* hdr_q;     // query-tile schedule (dQ)
  const WorkItem* items_q;
  const int32_t* order_q;
  const WsHeader* hdr_k;     // key-tile schedule (dK, dV)
  const WorkItem* items_k;
  const int32_t* order_k;
  int dkv_blocks;            // workgroups [0, dkv_blocks) run dK/dV tiles
};

struct MergeArgs {
  float* out;
  float* lse;
  const void* op;
  int64_t op_st, op_sh;
  const float* lsep;
  int64_t tokens;
  int heads;
  int d;
  int bf16;
};

struct DeltaArgs {
  const float* out;
  const void* dout;
  int64_t do_st, do_sh;
  float* delta;
  int64_t tokens;
  int heads;
  int d;
  int bf16;
};

struct PartArgs {
  const char* src;
  char* dst;
  int64_t src_st, src_sh, dst_st, dst_sh;  // strides in bytes
  const int32_t* cu;                        // global cu_seqlens
  int nseq;
  int64_t local_tokens;                     // upper bound on local rows (launch size)
  int64_t global_tokens;                    // rows of the global tensor
  int heads;
  int row_bytes;                            // head_dim * element size (multiple of 16)
  int cp, rank;
  int scatter;                              // 0: global -> local, 1: local -> global
  int tf_b, tf_n;                           // > 0: balanced teacher-forcing split
  int hw_h, hw_w, hw_sh, hw_sw;             // > 0: height/width split of frames x H x W tokens
  int cpr_shift;                            // log2(row_bytes / 16), set at launch
  int tok_per_block;                        // local rows per workgroup, set at launch
};

hipError_t launch_sched(const SchedArgs& a, hipStream_t stream);
hipError_t launch_sched_pair(const SchedArgs& a, const SchedArgs& b, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, bool bf16, int d, int64_t max_items, hipStream_t stream);
int fwd_tile_rows(bool bf16);
int bwd_dq_tile_rows(bool bf16);
int bwd_dkv_tile_rows(bool bf16);
hipError_t launch_bwd(BwdArgs a, bool bf16, int d, int64_t max_items_q, int64_t max_items_k, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_fill(float* dst, int64_t count, float value, hipStream_t stream);
hipError_t launch_delta(const DeltaArgs& a, hipStream_t stream);
hipError_t launch_partition(PartArgs a, hipStream_t stream);

// Copy of `tokens` rows x `heads` heads between two THD tensors, starting at
// (src_row0, src_h0) and (dst_row0, dst_h0): the one-device form of the
// Ulysses sequence<->head exchange.
struct HeadCopyArgs {
  const char* src;
  char* dst;
  int64_t src_st, src_sh, dst_st, dst_sh;   // strides in bytes
  int64_t src_row0, dst_row0, tokens;
  int src_h0, dst_h0, heads;
  int row_bytes;                            // head_dim * element size (multiple of 16)
};
hipError_t launch_head_copy(const HeadCopyArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Position in the unsplit sequence of local row `off` of a sequence whose
// local length is `len`, held by `rank` under the zigzag split: the local
// rows are [chunk rank ; chunk 2cp-1-rank], each len/2 long.
__device__ __forceinline__ int32_t zigzag_pos(int32_t off, int32_t len, int32_t cp, int32_t rank) {
  if (cp == 1) return off;
  int32_t c = len >> 1;
  return off < c ? rank * c + off : (2 * cp - 1 - rank) * c + (off - c);
}

// The mask predicate on in-sequence positions (query pq, key pk).
__host__ __device__ inline bool mask_allowed(int mode, int32_t pq, int32_t pk, int32_t tf_b, int32_t tf_n) {
  if (mode == CPATTN_MASK_CAUSAL) return pk <= pq;
  if (mode == CPATTN_MASK_BIDIR) return true;
  const int32_t span = tf_b * tf_n;
  const bool qn = pq >= span, kn = pk >= span;
  const int32_t cq = (qn ? pq - span : pq) / tf_b;
  const int32_t ck = (kn ? pk - span : pk) / tf_b;
  if (!qn) return !kn && ck <= cq;
  return kn ? ck == cq : ck < cq;
}

// The keys a query at position pq may attend, as at most two position
// intervals: p is allowed iff (unsigned)(p - lo1) < len1 or
// (unsigned)(p - lo2) < len2.  Same predicate as mask_allowed.
struct KeyRanges {
  unsigned lo1, len1, lo2, len2;
};

__host__ __device__ inline KeyRanges key_ranges(int mode, int32_t pq, int32_t tf_b, int32_t tf_n) {
  KeyRanges r;
  r.lo2 = 0u;
  r.len2 = 0u;
  if (mode == CPATTN_MASK_CAUSAL) {
    r.lo1 = 0u;
    r.len1 = (unsigned)(pq + 1);
  } else if (mode == CPATTN_MASK_BIDIR) {
    r.lo1 = 0u;
    r.len1 = 0xffffffffu;
  } else {
    const int32_t span = tf_b * tf_n;
    if (pq < span) {                      // clean chunk c: clean chunks <= c
      r.lo1 = 0u;
      r.len1 = (unsigned)((pq / tf_b + 1) * tf_b);
    } else {                              // noisy chunk c: clean < c, noisy == c
      const int32_t c = (pq - span) / tf_b;
      r.lo1 = 0u;
      r.len1 = (unsigned)(c * tf_b);
      r.lo2 = (unsigned)(span + c * tf_b);
      r.len2 = (unsigned)tf_b;
    }
  }
  return r;
}

// The queries that may attend a key at position pk (the transpose of
// key_ranges), as at most two position intervals.
__host__ __device__ inline KeyRanges query_ranges(int mode, int32_t pk, int32_t tf_b, int32_t tf_n) {
  KeyRanges r;
  r.lo2 = 0u;
  r.len2 = 0u;
  if (mode == CPATTN_MASK_CAUSAL) {
    r.lo1 = (unsigned)pk;
    r.len1 = 0x7fffffffu;
  } else if (mode == CPATTN_MASK_BIDIR) {
    r.lo1 = 0u;
    r.len1 = 0xffffffffu;
  } else {
    const int32_t span = tf_b * tf_n;
    if (pk < span) {                      // clean chunk c: clean >= c, noisy > c
      const int32_t c = pk / tf_b;
      r.lo1 = (unsigned)(c * tf_b);
      r.len1 = (unsigned)(span - c * tf_b);
      r.lo2 = (unsigned)(span + (c + 1) * tf_b);
      r.len2 = (unsigned)(span - (c + 1) * tf_b);
    } else {                              // noisy chunk c: noisy == c
      const int32_t c = (pk - span) / tf_b;
      r.lo1 = (unsigned)(span + c * tf_b);
      r.len1 = (unsigned)tf_b;
    }
  }
  return r;
}

__host__ __device__ inline bool in_ranges(const KeyRanges& r, int32_t pk) {
  return ((unsigned)pk - r.lo1 < r.len1) | ((unsigned)pk - r.lo2 < r.len2);
}

// A KeyRanges as two position windows [lo, end) with end saturated to
// INT_MAX.  For the intervals key_ranges and query_ranges produce (lo below
// 2^31, and lo = 0 whenever len exceeds 2^31) a position p >= 0 is allowed
// iff it lies in one of the windows: the same predicate as in_ranges.
struct KeyWindows {
  int lo1, end1, lo2, end2;
};

__host__ __device__ inline KeyWindows key_windows(const KeyRanges& r) {
  auto end = [](unsigned lo, unsigned len) {
    const unsigned long long e = (unsigned long long)lo + len;
    return e > 0x7fffffffull ? 0x7fffffff : (int)e;
  };
  return KeyWindows{(int)r.lo1, end(r.lo1, r.len1), (int)r.lo2, end(r.lo2, r.len2)};
}

// The predicate for the positions pbase + k, k < 28 (the offsets a lane's
// accumulator block holds), as a bit set: bit k is set iff k < rem and
// pbase + k lies in a window.  Each window becomes the offset range
// [lo - pbase, end - pbase) clipped to [0, min(rem, 28)), so a masked block
// costs one bit test per element instead of the range tests.
__host__ __device__ inline unsigned allowed_bits(const KeyWindows& w, int32_t pbase, int32_t rem) {
  const int lim = min(max(rem, 0), 28);
  auto window = [&](int lo, int end) {
    const int a = min(max(lo - pbase, 0), lim);
    const int b = min(max(end - pbase, a), lim);
    return ((1u << (b - a)) - 1u) << a;
  };
  return window(w.lo1, w.end1) | window(w.lo2, w.end2);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each index a constant
template <class F, int... I>
__device__ __forceinline__ void for_each_index_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void for_each_index(F&& f) {
  for_each_index_seq(f, std::make_integer_sequence<int, N>{});
}

// v where bit K of `bits` is set, else the bit pattern `off`: a
// sign-extended one-bit field and a bit-field select.
template <int K>
__device__ __forceinline__ float select_bit(unsigned bits, float v, unsigned off) {
  const unsigned m = (unsigned)__builtin_amdgcn_sbfe((int)bits, K, 1);
  return __uint_as_float((__float_as_uint(v) & m) | (off & ~m));
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace cpattn
