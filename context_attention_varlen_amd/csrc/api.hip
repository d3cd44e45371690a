// libcpattn C ABI: argument validation and dispatch.  Every entry point
// checks its arguments before anything is enqueued; no C++ exception leaves
// this file.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "common.h"

#define CPATTN_API extern "C" __attribute__((visibility("default")))

using namespace cpattn;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(cpattn_dtype t) { return t == CPATTN_BF16 ? 2 : 4; }

// A THD view the kernels can use: 16-byte aligned rows, head_dim 64 or 128.
cpattn_status check_tensor(const cpattn_tensor* t, bool need_data = true) {
  if (!t) return CPATTN_ERR_INVALID_ARG;
  if (t->dtype != CPATTN_F32 && t->dtype != CPATTN_BF16) return CPATTN_ERR_UNSUPPORTED;
  if (t->tokens < 0 || t->tokens >= kMaxRows || t->heads <= 0) return CPATTN_ERR_INVALID_ARG;
  if (t->head_dim != 64 && t->head_dim != 128) return CPATTN_ERR_UNSUPPORTED;
  if (need_data && t->tokens > 0 && (!t->data || !aligned16(t->data))) return CPATTN_ERR_INVALID_ARG;
  if (t->stride_token % 8 || t->stride_head % 8) return CPATTN_ERR_INVALID_ARG;
  // views whose (token, head) rows overlap are rejected: writes through
  // them would race
  if (t->heads > 1 && t->stride_head < t->head_dim) return CPATTN_ERR_INVALID_ARG;
  if (t->tokens > 1 && t->stride_token < (int64_t)(t->heads - 1) * t->stride_head + t->head_dim)
    return CPATTN_ERR_INVALID_ARG;
  return CPATTN_OK;
}

cpattn_status check_step(const cpattn_step* s, cpattn_mask_mode mode) {
  if (!s) return CPATTN_ERR_INVALID_ARG;
  if (s->cp < 1 || s->rank < 0 || s->rank >= s->cp || s->step < 0 || s->step >= s->cp)
    return CPATTN_ERR_INVALID_ARG;
  if (mode != CPATTN_MASK_CAUSAL && mode != CPATTN_MASK_BIDIR && mode != CPATTN_MASK_TF_BLOCK)
    return CPATTN_ERR_INVALID_ARG;
  if (mode == CPATTN_MASK_TF_BLOCK) {
    if (s->tf_chunk_tokens <= 0 || s->tf_num_chunks <= 0) return CPATTN_ERR_INVALID_ARG;
    if ((int64_t)s->tf_chunk_tokens * s->tf_num_chunks * 2 >= kMaxRows) return CPATTN_ERR_INVALID_ARG;
    // balanced split: equal time-chunk shares, and chunk blocks of at least
    // 32 rows (the workspace's item bound)
    if (s->cp > 1 && (s->tf_num_chunks % s->cp || s->tf_chunk_tokens < 32)) return CPATTN_ERR_INVALID_ARG;
  }
  return CPATTN_OK;
}

bool tf_split(cpattn_mask_mode mode, const cpattn_step* s) { return mode == CPATTN_MASK_TF_BLOCK && s->cp > 1; }

// Items a schedule over `tokens` primary rows can produce.
int64_t sched_items(cpattn_mask_mode mode, const cpattn_step* s, int64_t tokens, int32_t nseq, int tile) {
  if (tf_split(mode, s))
    return (int64_t)nseq * 2 * (s->tf_num_chunks / s->cp) * ((s->tf_chunk_tokens + tile - 1) / tile);
  return max_items_for(tokens, nseq, tile);
}

// Mask the attention kernels apply: under the balanced teacher-forcing split
// the scheduler hands them only fully allowed segments.
int kernel_mask(cpattn_mask_mode mode, const cpattn_step* s) {
  return tf_split(mode, s) ? (int)CPATTN_MASK_BIDIR : (int)mode;
}

int src_rank(const cpattn_step* s) { return ((s->rank - s->step) % s->cp + s->cp) % s->cp; }

thread_local char g_last_hip_error[256] = "";

cpattn_status hip_status(hipError_t e) {
  if (e == hipSuccess) return CPATTN_OK;
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%d)", hipGetErrorString(e), (int)e);
  return CPATTN_ERR_HIP;
}

// A runtime error left by an unrelated earlier call on this thread must not
// be reported as the failure of our launch: clear it before enqueueing.
void clear_stale_error() { (void)hipGetLastError(); }

// Host closed form: pairs (p, k), p in [a, a+C), k in [b, b+Cb), k <= p.
int64_t causal_block_pairs(int64_t a, int64_t C, int64_t b, int64_t Cb) {
  if (C <= 0 || Cb <= 0) return 0;
  auto F = [Cb](int64_t n) -> int64_t {  // sum_{y=1..n} min(y, Cb), 0 for n <= 0
    if (n <= 0) return 0;
    if (n <= Cb) return n * (n + 1) / 2;
    return Cb * (Cb + 1) / 2 + (n - Cb) * Cb;
  };
  const int64_t x0 = a - b + 1, x1 = a - b + C;
  return F(x1) - F(x0 - 1);
}

// Shared set-up of the scheduler arguments.
SchedArgs sched_args(void* ws, const int32_t* cu_p, const int32_t* cu_s, int nseq, int64_t tok_p,
                     int64_t tok_s, const cpattn_step* st, int rank_p, int rank_s, bool primary_is_q,
                     cpattn_mask_mode mode, int tile_p, int tile_s, int cost_mult, int64_t max_items,
                     const WsRegion& R) {
  SchedArgs a;
  a.cu_p = cu_p;
  a.cu_s = cu_s;
  a.nseq = nseq;
  a.tokens_p = tok_p;
  a.tokens_s = tok_s;
  a.cp = st->cp;
  a.rank_p = rank_p;
  a.rank_s = rank_s;
  a.primary_is_q = primary_is_q ? 1 : 0;
  a.mask = (int)mode;
  a.tf_b = mode == CPATTN_MASK_TF_BLOCK ? st->tf_chunk_tokens : 1;
  a.tf_n = mode == CPATTN_MASK_TF_BLOCK ? st->tf_num_chunks : 1;
  a.tile_p = tile_p;
  a.tile_s = tile_s;
  a.cost_mult = cost_mult;
  a.tail_items = 0;
  a.max_items = (int32_t)max_items;
  char* base = (char*)ws;
  a.hdr = (WsHeader*)(base + R.hdr);
  a.items = (WorkItem*)(base + R.items);
  a.order = (int32_t*)(base + R.order);
  a.seq_base = (int32_t*)(base + R.seq_base);
  return a;
}

}  // namespace

CPATTN_API const char* cpattn_version(void) { return "cpattn 0.1 (gfx950)"; }

CPATTN_API const char* cpattn_last_hip_error(void) { return g_last_hip_error; }

CPATTN_API cpattn_status cpattn_device_info(int32_t device, int32_t* cu_count, int32_t* clock_khz) {
  if (device < 0 || !cu_count || !clock_khz) return CPATTN_ERR_INVALID_ARG;
  int cus = 0, khz = 0;
  cpattn_status st;
  if ((st = hip_status(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device))) != CPATTN_OK)
    return st;
  if ((st = hip_status(hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device))) != CPATTN_OK) return st;
  *cu_count = cus;
  *clock_khz = khz;
  return CPATTN_OK;
}

CPATTN_API const char* cpattn_status_string(cpattn_status s) {
  switch (s) {
    case CPATTN_OK: return "ok";
    case CPATTN_ERR_INVALID_ARG: return "invalid argument";
    case CPATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case CPATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case CPATTN_ERR_HIP: return "HIP runtime error";
    case CPATTN_ERR_INFEASIBLE: return "no feasible plan";
    case CPATTN_ERR_NOMEM: return "out of host memory";
  }
  return "unknown status";
}

CPATTN_API cpattn_status cpattn_partition_index(const int32_t* cu_g, int32_t nseq, int32_t cp, int32_t rank,
                                                int32_t* cu_l, int64_t* l2g) {
  if (!cu_g || !cu_l || nseq < 0 || cp < 1 || rank < 0 || rank >= cp) return CPATTN_ERR_INVALID_ARG;
  if (cu_g[0] != 0) return CPATTN_ERR_INVALID_ARG;
  for (int b = 0; b < nseq; ++b) {
    const int64_t len = (int64_t)cu_g[b + 1] - cu_g[b];
    if (len < 0) return CPATTN_ERR_INVALID_ARG;
    if (cp > 1 && len % (2 * cp)) return CPATTN_ERR_INVALID_ARG;
  }
  cu_l[0] = 0;
  int64_t t = 0;
  for (int b = 0; b < nseq; ++b) {
    const int64_t g0 = cu_g[b], len = (int64_t)cu_g[b + 1] - g0;
    if (cp == 1) {
      if (l2g)
        for (int64_t o = 0; o < len; ++o) l2g[t + o] = g0 + o;
      t += len;
    } else {
      const int64_t C = len / (2 * cp);
      const int64_t chunks[2] = {rank, 2 * cp - 1 - rank};
      for (int h = 0; h < 2; ++h)
        for (int64_t o = 0; o < C; ++o) {
          if (l2g) l2g[t] = g0 + chunks[h] * C + o;
          ++t;
        }
    }
    cu_l[b + 1] = (int32_t)t;
  }
  return CPATTN_OK;
}

CPATTN_API cpattn_status cpattn_partition_index_tf(const int32_t* cu_g, int32_t nseq, int32_t cp, int32_t rank,
                                                   int32_t tf_chunk_tokens, int32_t tf_num_chunks, int32_t* cu_l,
                                                   int64_t* l2g) {
  if (!cu_g || !cu_l || nseq < 0 || cp < 1 || rank < 0 || rank >= cp) return CPATTN_ERR_INVALID_ARG;
  if (tf_chunk_tokens <= 0 || tf_num_chunks <= 0 || tf_num_chunks % cp || cu_g[0] != 0) return CPATTN_ERR_INVALID_ARG;
  const int64_t B = tf_chunk_tokens, N = tf_num_chunks, m = N / cp;
  for (int b = 0; b < nseq; ++b)
    if ((int64_t)cu_g[b + 1] - cu_g[b] != 2 * B * N) return CPATTN_ERR_INVALID_ARG;
  cu_l[0] = 0;
  int64_t t = 0;
  for (int b = 0; b < nseq; ++b) {
    const int64_t g0 = cu_g[b];
    for (int stream = 0; stream < 2; ++stream)
      for (int64_t k = 0; k < m; ++k) {
        const int64_t base = g0 + stream * B * N + (int64_t)tf_rank_chunk(rank, (int32_t)k, cp) * B;
        for (int64_t o = 0; o < B; ++o) {
          if (l2g) l2g[t] = base + o;
          ++t;
        }
      }
    cu_l[b + 1] = (int32_t)t;
  }
  return CPATTN_OK;
}

static cpattn_status partition_common(const cpattn_tensor* src, cpattn_tensor* dst, const int32_t* cu_dev,
                                      int32_t nseq, int32_t cp, int32_t rank, void* stream, bool scatter,
                                      int32_t tf_b = 0, int32_t tf_n = 0, const int32_t* hw = nullptr) {
  cpattn_status st;
  if ((st = check_tensor(src)) != CPATTN_OK) return st;
  if ((st = check_tensor(dst)) != CPATTN_OK) return st;
  if (!cu_dev || nseq < 0 || cp < 1 || rank < 0 || rank >= cp) return CPATTN_ERR_INVALID_ARG;
  if (src->dtype != dst->dtype || src->heads != dst->heads || src->head_dim != dst->head_dim)
    return CPATTN_ERR_INVALID_ARG;
  const cpattn_tensor* glob = scatter ? dst : src;
  const cpattn_tensor* loc = scatter ? src : dst;
  if (loc->tokens < glob->tokens / cp) return CPATTN_ERR_INVALID_ARG;
  const int es = elem_size(src->dtype);
  PartArgs a;
  a.src = (const char*)src->data;
  a.dst = (char*)dst->data;
  a.src_st = src->stride_token * es;
  a.src_sh = src->stride_head * es;
  a.dst_st = dst->stride_token * es;
  a.dst_sh = dst->stride_head * es;
  a.cu = cu_dev;
  a.nseq = nseq;
  a.local_tokens = glob->tokens / cp;
  a.global_tokens = glob->tokens;
  a.heads = src->heads;
  a.row_bytes = src->head_dim * es;
  a.cp = cp;
  a.rank = rank;
  a.scatter = scatter ? 1 : 0;
  a.tf_b = cp > 1 ? tf_b : 0;
  a.tf_n = cp > 1 ? tf_n : 0;
  a.hw_h = a.hw_w = a.hw_sh = a.hw_sw = 0;
  if (hw && cp > 1) {
    a.hw_h = hw[0];
    a.hw_w = hw[1];
    a.hw_sh = hw[2];
    a.hw_sw = hw[3];
  }
  clear_stale_error();
  return hip_status(launch_partition(a, (hipStream_t)stream));
}

CPATTN_API cpattn_status cpattn_partition(const cpattn_tensor* src_global, cpattn_tensor* dst_local,
                                          const int32_t* cu_dev, int32_t nseq, int32_t cp, int32_t rank,
                                          void* stream) {
  return partition_common(src_global, dst_local, cu_dev, nseq, cp, rank, stream, false);
}

CPATTN_API cpattn_status cpattn_unpartition(const cpattn_tensor* src_local, cpattn_tensor* dst_global,
                                            const int32_t* cu_dev, int32_t nseq, int32_t cp, int32_t rank,
                                            void* stream) {
  return partition_common(src_local, dst_global, cu_dev, nseq, cp, rank, stream, true);
}

CPATTN_API cpattn_status cpattn_partition_tf(const cpattn_tensor* src_global, cpattn_tensor* dst_local,
                                             const int32_t* cu_dev, int32_t nseq, int32_t cp, int32_t rank,
                                             int32_t tf_chunk_tokens, int32_t tf_num_chunks, void* stream) {
  if (tf_chunk_tokens <= 0 || tf_num_chunks <= 0 || tf_num_chunks % (cp > 0 ? cp : 1)) return CPATTN_ERR_INVALID_ARG;
  return partition_common(src_global, dst_local, cu_dev, nseq, cp, rank, stream, false, tf_chunk_tokens,
                          tf_num_chunks);
}

CPATTN_API cpattn_status cpattn_unpartition_tf(const cpattn_tensor* src_local, cpattn_tensor* dst_global,
                                               const int32_t* cu_dev, int32_t nseq, int32_t cp, int32_t rank,
                                               int32_t tf_chunk_tokens, int32_t tf_num_chunks, void* stream) {
  if (tf_chunk_tokens <= 0 || tf_num_chunks <= 0 || tf_num_chunks % (cp > 0 ? cp : 1)) return CPATTN_ERR_INVALID_ARG;
  return partition_common(src_local, dst_global, cu_dev, nseq, cp, rank, stream, true, tf_chunk_tokens,
                          tf_num_chunks);
}

// Shared checks and launches of the Ulysses exchange: shard s's rows sit at
// row offset sum_{s' < s} tokens(s') of the gathered tensor.
static cpattn_status ulysses_common(const cpattn_tensor* shards, int32_t n, int32_t group, const cpattn_tensor* g,
                                    void* stream, bool to_head) {
  cpattn_status st;
  if (!shards || !g || n < 1 || group < 0 || group >= n) return CPATTN_ERR_INVALID_ARG;
  if ((st = check_tensor(g)) != CPATTN_OK) return st;
  int64_t rows = 0;
  for (int s = 0; s < n; ++s) {
    if ((st = check_tensor(&shards[s])) != CPATTN_OK) return st;
    if (shards[s].dtype != g->dtype || shards[s].head_dim != g->head_dim || shards[s].heads != (int64_t)g->heads * n)
      return CPATTN_ERR_INVALID_ARG;
    rows += shards[s].tokens;
  }
  if (rows > g->tokens) return CPATTN_ERR_INVALID_ARG;
  const int es = elem_size(g->dtype);
  clear_stale_error();
  int64_t row0 = 0;
  for (int s = 0; s < n; ++s) {
    const cpattn_tensor& sh = shards[s];
    HeadCopyArgs a;
    const cpattn_tensor* src = to_head ? &sh : g;
    const cpattn_tensor* dst = to_head ? g : &sh;
    a.src = (const char*)src->data;
    a.dst = (char*)dst->data;
    a.src_st = src->stride_token * es;
    a.src_sh = src->stride_head * es;
    a.dst_st = dst->stride_token * es;
    a.dst_sh = dst->stride_head * es;
    a.src_row0 = to_head ? 0 : row0;
    a.dst_row0 = to_head ? row0 : 0;
    a.tokens = sh.tokens;
    a.src_h0 = to_head ? group * g->heads : 0;
    a.dst_h0 = to_head ? 0 : group * g->heads;
    a.heads = g->heads;
    a.row_bytes = g->head_dim * es;
    if ((st = hip_status(launch_head_copy(a, (hipStream_t)stream))) != CPATTN_OK) return st;
    row0 += sh.tokens;
  }
  return CPATTN_OK;
}

CPATTN_API cpattn_status cpattn_seq_to_head(const cpattn_tensor* shards, int32_t n_shards, int32_t group,
                                            cpattn_tensor* gathered, void* stream) {
  return ulysses_common(shards, n_shards, group, gathered, stream, true);
}

CPATTN_API cpattn_status cpattn_head_to_seq(const cpattn_tensor* gathered, int32_t n_shards, int32_t group,
                                            cpattn_tensor* shards, void* stream) {
  return ulysses_common(shards, n_shards, group, gathered, stream, false);
}

// ---- height/width split (LongCat-Video context-parallel page) -------------
static bool hw_valid(int32_t frames, int32_t H, int32_t W, int32_t sh, int32_t sw) {
  return frames > 0 && H > 0 && W > 0 && sh > 0 && sw > 0 && H % sh == 0 && W % sw == 0 &&
         (int64_t)frames * H * W < kMaxRows;
}

CPATTN_API cpattn_status cpattn_split_hw(int32_t H, int32_t W, int32_t cp, int32_t* split_h, int32_t* split_w) {
  if (H <= 0 || W <= 0 || cp < 1 || !split_h || !split_w) return CPATTN_ERR_INVALID_ARG;
  int best_h = 0;
  double best = 0.0;
  for (int a = 1; a <= cp; ++a) {
    if (cp % a || H % a || W % (cp / a)) continue;
    const double d = std::fabs((double)H / a - (double)W / (cp / a));
    if (best_h == 0 || d < best) {   // ascending a: ties keep the smaller height split
      best_h = a;
      best = d;
    }
  }
  if (best_h == 0) return CPATTN_ERR_INVALID_ARG;
  *split_h = best_h;
  *split_w = cp / best_h;
  return CPATTN_OK;
}

CPATTN_API cpattn_status cpattn_partition_index_hw(const int32_t* cu_g, int32_t nseq, int32_t frames, int32_t H,
                                                   int32_t W, int32_t split_h, int32_t split_w, int32_t rank,
                                                   int32_t* cu_l, int64_t* l2g) {
  if (!cu_g || !cu_l || nseq < 0 || !hw_valid(frames, H, W, split_h, split_w) || cu_g[0] != 0)
    return CPATTN_ERR_INVALID_ARG;
  const int32_t cp = split_h * split_w;
  if (rank < 0 || rank >= cp) return CPATTN_ERR_INVALID_ARG;
  const int64_t L = (int64_t)frames * H * W, th = H / split_h, tw = W / split_w;
  const int64_t rh = rank / split_w, rw = rank % split_w;
  for (int b = 0; b < nseq; ++b)
    if ((int64_t)cu_g[b + 1] - cu_g[b] != L) return CPATTN_ERR_INVALID_ARG;
  cu_l[0] = 0;
  int64_t t = 0;
  for (int b = 0; b < nseq; ++b) {
    for (int64_t f = 0; f < frames; ++f)
      for (int64_t h = rh * th; h < (rh + 1) * th; ++h)
        for (int64_t w = rw * tw; w < (rw + 1) * tw; ++w) {
          if (l2g) l2g[t] = cu_g[b] + (f * H + h) * W + w;
          ++t;
        }
    cu_l[b + 1] = (int32_t)t;
  }
  return CPATTN_OK;
}

CPATTN_API cpattn_status cpattn_partition_hw(const cpattn_tensor* src_global, cpattn_tensor* dst_local,
                                             const int32_t* cu_dev, int32_t nseq, int32_t frames, int32_t H,
                                             int32_t W, int32_t split_h, int32_t split_w, int32_t rank,
                                             void* stream) {
  if (!hw_valid(frames, H, W, split_h, split_w)) return CPATTN_ERR_INVALID_ARG;
  const int32_t hw[4] = {H, W, split_h, split_w};
  return partition_common(src_global, dst_local, cu_dev, nseq, split_h * split_w, rank, stream, false, 0, 0, hw);
}

CPATTN_API cpattn_status cpattn_unpartition_hw(const cpattn_tensor* src_local, cpattn_tensor* dst_global,
                                               const int32_t* cu_dev, int32_t nseq, int32_t frames, int32_t H,
                                               int32_t W, int32_t split_h, int32_t split_w, int32_t rank,
                                               void* stream) {
  if (!hw_valid(frames, H, W, split_h, split_w)) return CPATTN_ERR_INVALID_ARG;
  const int32_t hw[4] = {H, W, split_h, split_w};
  return partition_common(src_local, dst_global, cu_dev, nseq, split_h * split_w, rank, stream, true, 0, 0, hw);
}

CPATTN_API int64_t cpattn_count_pairs(const int32_t* cu_g, int32_t nseq, cpattn_mask_mode mode,
                                      const cpattn_step* st) {
  if (!cu_g || nseq < 0 || check_step(st, mode) != CPATTN_OK || cu_g[0] != 0) return -1;
  const int cp = st->cp, r = st->rank, j = src_rank(st);
  int64_t total = 0;
  for (int b = 0; b < nseq; ++b) {
    const int64_t L = (int64_t)cu_g[b + 1] - cu_g[b];
    if (L < 0 || (cp > 1 && L % (mode == CPATTN_MASK_BIDIR ? cp : 2 * cp))) return -1;
    if (mode == CPATTN_MASK_TF_BLOCK) {
      const int64_t B = st->tf_chunk_tokens, N = st->tf_num_chunks;
      if (L != 2 * B * N) return -1;
      if (cp == 1) {
        total += N * (N + 1) * B * B;
        continue;
      }
      // balanced split: rank r's clean query chunk c sees source j's clean
      // chunks <= c, its noisy chunk c sees j's clean chunks < c plus the
      // noisy chunk c when j holds it
      for (int32_t k = 0; k < N / cp; ++k) {
        const int32_t c = tf_rank_chunk(r, k, cp);
        total += B * B * (tf_count_below(j, c + 1, cp) + tf_count_below(j, c, cp) + (tf_owner(c, cp) == j ? 1 : 0));
      }
      continue;
    }
    if (cp == 1) {
      total += mode == CPATTN_MASK_BIDIR ? L * L : causal_block_pairs(0, L, 0, L);
      continue;
    }
    if (mode == CPATTN_MASK_BIDIR) {    // any split: every local query sees every local key of the source
      total += (L / cp) * (L / cp);
      continue;
    }
    const int64_t C = L / (2 * cp);
    const int64_t qc[2] = {r, 2 * cp - 1 - r}, kc[2] = {j, 2 * cp - 1 - j};
    for (int x = 0; x < 2; ++x)
      for (int y = 0; y < 2; ++y)
        total += mode == CPATTN_MASK_BIDIR ? C * C : causal_block_pairs(qc[x] * C, C, kc[y] * C, C);
  }
  return total;
}

CPATTN_API int32_t cpattn_step_source(const cpattn_step* st) {
  if (!st || st->cp < 1 || st->rank < 0 || st->rank >= st->cp || st->step < 0 || st->step >= st->cp) return -1;
  return src_rank(st);
}

CPATTN_API size_t cpattn_workspace_size(int64_t tokens_q, int64_t tokens_k, int32_t nseq) {
  if (tokens_q < 0 || tokens_k < 0 || nseq < 0) return 0;
  return ws_layout(tokens_q, tokens_k, nseq).total;
}

CPATTN_API cpattn_status cpattn_workspace_status(const void* ws, void* stream, cpattn_status* out) {
  if (!ws || !out) return CPATTN_ERR_INVALID_ARG;
  cpattn_status st;
  if ((st = hip_status(hipStreamSynchronize((hipStream_t)stream))) != CPATTN_OK) return st;
  int32_t v = 0;
  if ((st = hip_status(hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost))) != CPATTN_OK) return st;
  *out = (cpattn_status)v;
  return CPATTN_OK;
}

static cpattn_status fwd_step_impl(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                   const int32_t* cu_q, const int32_t* cu_k, int32_t nseq, cpattn_mask_mode mode,
                                   const cpattn_step* step, float scale, cpattn_tensor* out, float* lse, void* ws,
                                   size_t ws_bytes, void* stream) {
  cpattn_status st;
  if ((st = check_tensor(q)) || (st = check_tensor(k)) || (st = check_tensor(v)) || (st = check_tensor(out)))
    return st;
  if ((st = check_step(step, mode)) != CPATTN_OK) return st;
  if (q->dtype != k->dtype || q->dtype != v->dtype || q->dtype != out->dtype) return CPATTN_ERR_INVALID_ARG;
  if (q->head_dim != k->head_dim || q->head_dim != v->head_dim || q->head_dim != out->head_dim)
    return CPATTN_ERR_INVALID_ARG;
  if (k->heads != v->heads || q->heads != out->heads || q->heads % k->heads) return CPATTN_ERR_INVALID_ARG;
  if (q->tokens != out->tokens || k->tokens != v->tokens) return CPATTN_ERR_INVALID_ARG;
  if (!cu_q || !cu_k || nseq < 0 || (!lse && q->tokens > 0) || (lse && !aligned16(lse)))
    return CPATTN_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(q->tokens, k->tokens, nseq);
  if (!ws || ws_bytes < L.total || !aligned16(ws)) return CPATTN_ERR_WORKSPACE;

  const bool bf16 = q->dtype == CPATTN_BF16;
  const int d = q->head_dim;
  const int tile_p = fwd_tile_rows(bf16);
  // rows past cu_seqlens_q[nseq] (a padded buffer) get items with no keys,
  // so every row of out_partial / lse_partial is written; the zigzag bound
  // already counts them, the teacher-forcing one does not
  const int64_t max_items = sched_items(mode, step, q->tokens, nseq, tile_p) +
                            (tf_split(mode, step) ? (q->tokens + tile_p - 1) / tile_p : 0);
  if (max_items > ws_item_capacity(q->tokens, nseq)) return CPATTN_ERR_INVALID_ARG;
  SchedArgs sa = sched_args(ws, cu_q, cu_k, nseq, q->tokens, k->tokens, step, step->rank, src_rank(step),
                            true, mode, tile_p, 64, 1, max_items, L.a);
  sa.tail_items = 1;
  hipStream_t s = (hipStream_t)stream;
  clear_stale_error();
  if ((st = hip_status(launch_sched(sa, s))) != CPATTN_OK) return st;
  if (q->tokens == 0) return CPATTN_OK;

  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  FwdArgs a;
  a.q = q->data;
  a.k = k->data;
  a.v = v->data;
  a.q_st = q->stride_token; a.q_sh = q->stride_head;
  a.k_st = k->stride_token; a.k_sh = k->stride_head;
  a.v_st = v->stride_token; a.v_sh = v->stride_head;
  a.out = out->data;
  a.o_st = out->stride_token; a.o_sh = out->stride_head;
  a.lse = lse;
  a.tq = q->tokens;
  a.hq = q->heads;
  a.hkv = k->heads;
  a.grp = q->heads / k->heads;
  a.scale = sc;
  a.scale_log2 = sc * 1.4426950408889634f;
  a.mask = kernel_mask(mode, step);
  a.tf_b = sa.tf_b;
  a.tf_n = sa.tf_n;
  a.hdr = sa.hdr;
  a.items = sa.items;
  a.order = sa.order;
  return hip_status(launch_fwd(a, bf16, d, max_items, s));
}

CPATTN_API cpattn_status cpattn_fwd_step(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                         const int32_t* cu_q, const int32_t* cu_k, int32_t nseq,
                                         cpattn_mask_mode mode, const cpattn_step* step, float scale,
                                         cpattn_tensor* out, float* lse, void* ws, size_t ws_bytes,
                                         void* stream) {
  return fwd_step_impl(q, k, v, cu_q, cu_k, nseq, mode, step, scale, out, lse, ws, ws_bytes, stream);
}

// ---- allocation-free forward step ------------------------------------------
// The schedule workspace of cpattn_fwd_step_noalloc lives in this file-scope
// device array; every GPU the library runs on holds its own copy for the
// life of the process.  In host code `scratch` only names the symbol: its
// device address on the current GPU comes from hipGetSymbolAddress, resolved
// once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[CPATTN_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

cpattn_status scratch_ptr(void** out) {
  int dev = -1;
  cpattn_status st;
  if ((st = hip_status(hipGetDevice(&dev))) != CPATTN_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return CPATTN_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      // the device that is current now is the one whose copy is resolved
      if ((st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))) != CPATTN_OK) return st;
      if (!p) return CPATTN_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CPATTN_OK;
}

}  // namespace

CPATTN_API cpattn_status cpattn_fwd_step_noalloc(const cpattn_tensor* q, const cpattn_tensor* k,
                                                 const cpattn_tensor* v, const int32_t* cu_q, const int32_t* cu_k,
                                                 int32_t nseq, cpattn_mask_mode mode, const cpattn_step* step,
                                                 float scale, cpattn_tensor* out, float* lse, void* stream) {
  // size check first: a shape beyond the array is refused before any HIP call
  if (!q || !k || q->tokens < 0 || k->tokens < 0 || nseq < 0) return CPATTN_ERR_INVALID_ARG;
  if (ws_layout(q->tokens, k->tokens, nseq).total > (size_t)CPATTN_SCRATCH_BYTES) return CPATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  cpattn_status st;
  if ((st = scratch_ptr(&ws)) != CPATTN_OK) return st;
  return fwd_step_impl(q, k, v, cu_q, cu_k, nseq, mode, step, scale, out, lse, ws, CPATTN_SCRATCH_BYTES, stream);
}

CPATTN_API cpattn_status cpattn_merge(float* out, float* lse, const cpattn_tensor* op, const float* lsep,
                                      void* stream) {
  cpattn_status st;
  if ((st = check_tensor(op)) != CPATTN_OK) return st;
  if (op->tokens > 0 && (!out || !lse || !lsep || !aligned16(out))) return CPATTN_ERR_INVALID_ARG;
  MergeArgs a;
  a.out = out;
  a.lse = lse;
  a.op = op->data;
  a.op_st = op->stride_token;
  a.op_sh = op->stride_head;
  a.lsep = lsep;
  a.tokens = op->tokens;
  a.heads = op->heads;
  a.d = op->head_dim;
  a.bf16 = op->dtype == CPATTN_BF16;
  clear_stale_error();
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

CPATTN_API cpattn_status cpattn_fill_f32(float* dst, int64_t count, float value, void* stream) {
  if (count < 0 || (count > 0 && (!dst || !aligned16(dst)))) return CPATTN_ERR_INVALID_ARG;
  if (count == 0) return CPATTN_OK;
  clear_stale_error();
  return hip_status(launch_fill(dst, count, value, (hipStream_t)stream));
}

CPATTN_API cpattn_status cpattn_bwd_preprocess(const float* out, const cpattn_tensor* dout, float* delta,
                                               void* stream) {
  cpattn_status st;
  if ((st = check_tensor(dout)) != CPATTN_OK) return st;
  if (dout->tokens > 0 && (!out || !delta || !aligned16(out))) return CPATTN_ERR_INVALID_ARG;
  DeltaArgs a;
  a.out = out;
  a.dout = dout->data;
  a.do_st = dout->stride_token;
  a.do_sh = dout->stride_head;
  a.delta = delta;
  a.tokens = dout->tokens;
  a.heads = dout->heads;
  a.d = dout->head_dim;
  a.bf16 = dout->dtype == CPATTN_BF16;
  clear_stale_error();
  return hip_status(launch_delta(a, (hipStream_t)stream));
}

CPATTN_API cpattn_status cpattn_bwd_step(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                         const cpattn_tensor* dout, const float* lse, const float* delta,
                                         const int32_t* cu_q, const int32_t* cu_k, int32_t nseq,
                                         cpattn_mask_mode mode, const cpattn_step* step, float scale, float* dq,
                                         float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
  cpattn_status st;
  if ((st = check_tensor(q)) || (st = check_tensor(k)) || (st = check_tensor(v)) || (st = check_tensor(dout)))
    return st;
  if ((st = check_step(step, mode)) != CPATTN_OK) return st;
  if (q->dtype != k->dtype || q->dtype != v->dtype || q->dtype != dout->dtype) return CPATTN_ERR_INVALID_ARG;
  if (q->head_dim != k->head_dim || q->head_dim != v->head_dim || q->head_dim != dout->head_dim)
    return CPATTN_ERR_INVALID_ARG;
  if (k->heads != v->heads || q->heads != dout->heads || q->heads % k->heads) return CPATTN_ERR_INVALID_ARG;
  if (q->tokens != dout->tokens || k->tokens != v->tokens) return CPATTN_ERR_INVALID_ARG;
  if (!cu_q || !cu_k || nseq < 0) return CPATTN_ERR_INVALID_ARG;
  if (q->tokens > 0 && (!lse || !delta || !dq || !aligned16(dq))) return CPATTN_ERR_INVALID_ARG;
  if (k->tokens > 0 && (!dk || !dv || !aligned16(dk) || !aligned16(dv))) return CPATTN_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(q->tokens, k->tokens, nseq);
  if (!ws || ws_bytes < L.total || !aligned16(ws)) return CPATTN_ERR_WORKSPACE;

  const bool bf16 = q->dtype == CPATTN_BF16;
  const int d = q->head_dim;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  const int grp = q->heads / k->heads;
  hipStream_t s = (hipStream_t)stream;

  BwdArgs a;
  a.q = q->data; a.k = k->data; a.v = v->data; a.dout = dout->data;
  a.q_st = q->stride_token; a.q_sh = q->stride_head;
  a.k_st = k->stride_token; a.k_sh = k->stride_head;
  a.v_st = v->stride_token; a.v_sh = v->stride_head;
  a.do_st = dout->stride_token; a.do_sh = dout->stride_head;
  a.lse = lse; a.delta = delta; a.tq = q->tokens;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.hq = q->heads; a.hkv = k->heads; a.grp = grp;
  a.scale = sc; a.scale_log2 = sc * 1.4426950408889634f;
  a.mask = kernel_mask(mode, step);

  // schedules: query tiles (dQ) in region A, key tiles (dK, dV; cost counts
  // every q-head of the group) in region B
  const int tq = bwd_dq_tile_rows(bf16), tk = bwd_dkv_tile_rows(bf16);
  const int64_t mq = sched_items(mode, step, q->tokens, nseq, tq), mk = sched_items(mode, step, k->tokens, nseq, tk);
  if (mq > ws_item_capacity(q->tokens, nseq) || mk > ws_item_capacity(k->tokens, nseq)) return CPATTN_ERR_INVALID_ARG;
  const SchedArgs sq = sched_args(ws, cu_q, cu_k, nseq, q->tokens, k->tokens, step, step->rank, src_rank(step),
                                  true, mode, tq, 64, 1, mq, L.a);
  const SchedArgs sk = sched_args(ws, cu_k, cu_q, nseq, k->tokens, q->tokens, step, src_rank(step), step->rank,
                                  false, mode, tk, 64, grp, mk, L.b);
  a.tf_b = sq.tf_b; a.tf_n = sq.tf_n;
  a.hdr_q = sq.hdr; a.items_q = sq.items; a.order_q = sq.order;
  a.hdr_k = sk.hdr; a.items_k = sk.items; a.order_k = sk.order;
  clear_stale_error();
  if ((st = hip_status(launch_sched_pair(sq, sk, s))) != CPATTN_OK) return st;
  if (nseq == 0 || q->tokens == 0 || k->tokens == 0) return CPATTN_OK;
  return hip_status(launch_bwd(a, bf16, d, mq, mk, s));
}
