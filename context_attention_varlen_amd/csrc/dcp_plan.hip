// Dynamic-CP microbatch planner (host only): packs a global batch of
// variable-length samples into microbatches, gives each microbatch a
// power-of-two context-parallel size and places it on the rank x slot grid.
//
// "Speeding up Variable-Length Training with Dynamic Context Parallelism and
// NVIDIA Megatron Core", section A2 (data scheduling model, Eq. 1-3) and
// section A7 (zero-overhead runtime, Fig. 7).  The page gives the pieces in
// words only; the readings used here:
//   workload   w(S) = a S^2 + b S; memory: tokens per rank, S for cp = 1,
//              else S rounded up to 2c equal zigzag chunks, over c.
//   quota      Eq. 1-3 with all ranks at m microbatches: W = total/(gpus m).
//   stage 1    a sample gets the smallest power-of-two cp size whose share
//              meets the quota and the memory cap (max_cp when no size meets
//              the quota); a sample with cp > 1 opens its own microbatch.
//   stage 2    those microbatches, heaviest first, are topped up with the
//              lightest cp = 1 samples while quota and cap hold.
//   stage 3    the remaining samples, heaviest first, go to the least-loaded
//              cp = 1 microbatch with memory for them; there are as many
//              as grid cells left over.
//   placement  split microbatches (largest cp first) on the free aligned
//              group of least load, cp = 1 ones on the least-loaded rank.
//   simulator  rank time V * sum(slot loads) + (p - 1) * max(slot load);
//              step time = slowest rank.
//   search     m over [m_min, m_max] within a radius of the knee of the
//              budget curve (farthest point below the chord of the
//              normalised curve, Satopaa et al. 2011); least step time wins.
// Every decision but the knee compares exact integers (128-bit); the knee
// compares IEEE doubles, with contraction off so the rounding is the plain
// sequence of operations written here.  Ties go to the lower index.

#include "common.h"

#include <algorithm>
#include <cmath>
#include <queue>
#include <vector>

#pragma clang fp contract(off)

#define CPATTN_API extern "C" __attribute__((visibility("default")))

namespace cpattn {
namespace {

typedef __int128 i128;

struct Sample { int64_t len; i128 w; };

struct Mb {
  int32_t cp;
  i128 load;          // sum of w(S)
  int64_t tokens;     // per rank
  int32_t slot, rank; // rank = first rank of the group
  int32_t first;      // index of the sample that opened it (-1: none)
};

struct Plan {
  std::vector<Mb> mbs;          // split microbatches first, then cp = 1 ones
  std::vector<int32_t> owner;   // sample -> microbatch
  i128 time;
};

int64_t rank_tokens(int64_t S, int32_t c) {
  if (c == 1) return S;
  const int64_t chunk = (S + 2 * c - 1) / (2 * c);
  return 2 * chunk;
}

class Planner {
 public:
  Planner(const int32_t* lengths, int32_t n, const cpattn_dcp_config& cfg) : cfg_(cfg) {
    s_.resize(n);
    total_ = 0;
    wmax_ = 0;
    for (int32_t i = 0; i < n; ++i) {
      const int64_t S = lengths[i];
      s_[i] = {S, (i128)cfg.work_quad * S * S + (i128)cfg.work_lin * S};
      total_ += s_[i].w;
      wmax_ = std::max(wmax_, s_[i].w);
    }
    // the two orders every m uses: workload descending and ascending, both
    // with ties by index ascending
    desc_.resize(n);
    for (int32_t i = 0; i < n; ++i) desc_[i] = i;
    asc_ = desc_;
    std::sort(desc_.begin(), desc_.end(), [&](int32_t a, int32_t b) {
      return s_[a].w != s_[b].w ? s_[a].w > s_[b].w : a < b;
    });
    std::sort(asc_.begin(), asc_.end(), [&](int32_t a, int32_t b) {
      return s_[a].w != s_[b].w ? s_[a].w < s_[b].w : a < b;
    });
  }

  i128 total() const { return total_; }
  i128 wmax() const { return wmax_; }

  // Stage 1 cp size, or 0 when no size up to max_cp fits the memory cap.
  int32_t pick_cp(const Sample& x, int32_t m) const {
    const i128 gm = (i128)cfg_.gpus * m;
    for (int32_t c = 1;; c *= 2) {
      const bool mem_ok = rank_tokens(x.len, c) <= cfg_.mem_tokens;
      const bool quota_ok = x.w * gm <= (i128)c * total_;
      if (mem_ok && (quota_ok || c == cfg_.max_cp)) return c;
      if (c == cfg_.max_cp) return 0;
    }
  }

  bool build(int32_t m, Plan& p) const {
    const int32_t n = (int32_t)s_.size();
    const i128 gm = (i128)cfg_.gpus * m;
    std::vector<int32_t> cps(n);
    for (int32_t i = 0; i < n; ++i) {
      cps[i] = pick_cp(s_[i], m);
      if (cps[i] == 0) return false;
    }
    std::vector<int32_t> heavy, light;   // heaviest first; lightest first
    for (int32_t i : desc_)
      if (cps[i] > 1) heavy.push_back(i);
    for (int32_t i : asc_)
      if (cps[i] == 1) light.push_back(i);
    p.mbs.clear();
    p.owner.assign(n, -1);
    // stage 1: one microbatch per split sample, heaviest first
    int64_t split_cells = 0;
    for (int32_t i : heavy) {
      Mb mb{cps[i], s_[i].w, rank_tokens(s_[i].len, cps[i]), -1, -1, i};
      p.owner[i] = (int32_t)p.mbs.size();
      p.mbs.push_back(mb);
      split_cells += cps[i];
    }
    // stage 2: top up with the lightest cp = 1 samples (ascending workload)
    size_t next = 0;
    for (size_t j = 0; j < p.mbs.size() && next < light.size(); ++j) {
      Mb& mb = p.mbs[j];
      while (next < light.size()) {
        const Sample& x = s_[light[next]];
        const int64_t t = rank_tokens(x.len, mb.cp);
        if ((mb.load + x.w) * gm > (i128)mb.cp * total_ || mb.tokens + t > cfg_.mem_tokens) break;
        mb.load += x.w;
        mb.tokens += t;
        p.owner[light[next]] = (int32_t)j;
        ++next;
      }
    }
    // stage 3: the rest, heaviest first, to the least-loaded cp = 1 microbatch
    const int64_t ones = (int64_t)gm - split_cells;
    if (ones < 0) return false;
    const size_t base = p.mbs.size();
    for (int64_t j = 0; j < ones; ++j) p.mbs.push_back(Mb{1, 0, 0, -1, -1, -1});
    // the unsplit samples stage 2 left, heaviest first
    std::vector<int32_t> rest;
    for (int32_t i : desc_)
      if (cps[i] == 1 && p.owner[i] < 0) rest.push_back(i);
    if (!rest.empty() && ones == 0) return false;
    // Min-heap on (load, index).  A microbatch popped without room for the
    // current sample is parked by its free room; samples come longest first,
    // so it rejoins the heap only once a sample fits that room.  The heap
    // top is then always the least-loaded microbatch with room.
    typedef std::pair<i128, int32_t> Key;
    std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
    for (int64_t j = 0; j < ones; ++j) heap.push(Key(0, (int32_t)(base + j)));
    std::priority_queue<std::pair<int64_t, int32_t>> parked;   // (free room, index), largest room first
    for (int32_t i : rest) {
      const Sample& x = s_[i];
      while (!parked.empty() && parked.top().first >= x.len) {
        const int32_t b = parked.top().second;
        parked.pop();
        heap.push(Key(p.mbs[b].load, b));
      }
      int32_t hit = -1;
      while (!heap.empty()) {
        const Key k = heap.top();
        heap.pop();
        const int64_t room = cfg_.mem_tokens - p.mbs[k.second].tokens;
        if (room >= x.len) { hit = k.second; break; }
        parked.push(std::make_pair(room, k.second));
      }
      if (hit < 0) return false;
      Mb& mb = p.mbs[hit];
      mb.load += x.w;
      mb.tokens += x.len;
      p.owner[i] = hit;
      heap.push(Key(mb.load, hit));
    }
    return place(p, m, base);
  }

  i128 simulate(const Plan& p) const {
    const int32_t G = cfg_.gpus;
    std::vector<i128> sum(G, 0), mx(G, 0);
    for (const Mb& mb : p.mbs) {
      const i128 share = mb.load * (cfg_.max_cp / mb.cp);
      for (int32_t r = mb.rank; r < mb.rank + mb.cp; ++r) {
        sum[r] += share;
        mx[r] = std::max(mx[r], share);
      }
    }
    i128 t = 0;
    for (int32_t r = 0; r < G; ++r) t = std::max(t, (i128)cfg_.vpp * sum[r] + (i128)(cfg_.pp - 1) * mx[r]);
    return t;
  }

 private:
  bool place(Plan& p, int32_t m, size_t base) const {
    const int32_t G = cfg_.gpus;
    std::vector<uint8_t> used((size_t)G * m, 0);     // [slot][rank]
    std::vector<i128> load(G, 0);
    std::vector<size_t> order(base);
    for (size_t j = 0; j < base; ++j) order[j] = j;
    std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
      const Mb &x = p.mbs[a], &y = p.mbs[b];
      if (x.cp != y.cp) return x.cp > y.cp;
      if (x.load != y.load) return x.load > y.load;
      return x.first < y.first;
    });
    // The choice is the least (max rank load of the group, slot, group)
    // over every aligned group with a free slot.  Split microbatches come
    // largest cp first, so the taken cells of a slot form aligned blocks at
    // least as large as the current one: an aligned block of the current
    // size is wholly free or wholly taken, its first cell tells which, and a
    // group's best slot is its lowest free one (a pointer that only moves up
    // while the size stays the same).
    int32_t cur_c = 0;
    std::vector<int32_t> group_free;
    for (size_t j : order) {
      Mb& mb = p.mbs[j];
      const int32_t c = mb.cp, ng = G / c;
      if (c != cur_c) {
        cur_c = c;
        group_free.assign(ng, 0);
      }
      int32_t bg = -1, bk = 0;
      i128 best = 0;
      for (int32_t g = 0; g < ng; ++g) {
        int32_t& k = group_free[g];
        while (k < m && used[(size_t)k * G + (size_t)g * c]) ++k;
        if (k == m) continue;
        i128 mxl = 0;
        for (int32_t r = g * c; r < (g + 1) * c; ++r) mxl = std::max(mxl, load[r]);
        if (bg < 0 || mxl < best || (mxl == best && k < bk)) {
          bg = g;
          bk = k;
          best = mxl;
        }
      }
      if (bg < 0) return false;
      mb.slot = bk;
      mb.rank = bg * c;
      const i128 share = mb.load * (cfg_.max_cp / c);
      for (int32_t r = bg * c; r < (bg + 1) * c; ++r) {
        used[(size_t)bk * G + r] = 1;
        load[r] += share;
      }
    }
    // cp = 1 microbatches, heaviest first, on the least-loaded rank that has
    // a free slot (its lowest free slot)
    std::vector<size_t> ones;
    for (size_t j = base; j < p.mbs.size(); ++j) ones.push_back(j);
    std::stable_sort(ones.begin(), ones.end(), [&](size_t a, size_t b) { return p.mbs[a].load > p.mbs[b].load; });
    std::vector<int32_t> next_free(G, 0);
    auto advance = [&](int32_t r) {
      while (next_free[r] < m && used[(size_t)next_free[r] * G + r]) ++next_free[r];
    };
    typedef std::pair<i128, int32_t> Key;
    std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
    for (int32_t r = 0; r < G; ++r) {
      advance(r);
      if (next_free[r] < m) heap.push(Key(load[r], r));
    }
    for (size_t j : ones) {
      if (heap.empty()) return false;
      const int32_t r = heap.top().second;
      heap.pop();
      Mb& mb = p.mbs[j];
      mb.slot = next_free[r];
      mb.rank = r;
      used[(size_t)mb.slot * G + r] = 1;
      load[r] += mb.load * cfg_.max_cp;
      advance(r);
      if (next_free[r] < m) heap.push(Key(load[r], r));
    }
    return true;
  }

  cpattn_dcp_config cfg_;
  std::vector<Sample> s_;
  std::vector<int32_t> desc_, asc_;
  i128 total_, wmax_;
};

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace
}  // namespace cpattn

using namespace cpattn;

CPATTN_API cpattn_status cpattn_dcp_quotas(const int32_t* m, int32_t n, int32_t vpp, int32_t pp, double total,
                                           double* W) {
  if (!m || !W || n < 1 || vpp < 1 || pp < 1 || !(total >= 0.0) || !std::isfinite(total))
    return CPATTN_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (m[i] < 1) return CPATTN_ERR_INVALID_ARG;
  // Eq. 1: W_i (m_i V + p - 1) = K on every rank; Eq. 3: sum_i W_i m_i = total
  double inv = 0.0;
  for (int32_t i = 0; i < n; ++i) inv += (double)m[i] / ((double)m[i] * vpp + (pp - 1));
  const double K = total / inv;
  for (int32_t i = 0; i < n; ++i) W[i] = K / ((double)m[i] * vpp + (pp - 1));
  return CPATTN_OK;
}

static cpattn_status plan_batch(const int32_t* lengths, int32_t n, const cpattn_dcp_config& c, int32_t nm,
                                cpattn_dcp_plan* out);

CPATTN_API cpattn_status cpattn_dcp_plan_batch(const int32_t* lengths, int32_t n, const cpattn_dcp_config* cfg,
                                               cpattn_dcp_plan* out) {
  if (!lengths || !cfg || !out || n < 1 || n > (1 << 24)) return CPATTN_ERR_INVALID_ARG;
  const cpattn_dcp_config& c = *cfg;
  if (c.gpus < 1 || c.gpus > 65536 || !is_pow2(c.max_cp) || c.max_cp > c.gpus || c.gpus % c.max_cp ||
      c.pp < 1 || c.pp > 4096 || c.vpp < 1 || c.vpp > 4096 || c.mem_tokens < 1 ||
      c.work_quad < 0 || c.work_quad > (1 << 16) || c.work_lin < 0 || c.work_lin > (int64_t(1) << 32) ||
      c.work_quad + c.work_lin == 0 || c.m_min < 1 || c.m_max < c.m_min || c.m_max > 4096 ||
      (int64_t)c.gpus * c.m_max > (1 << 22))
    return CPATTN_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (lengths[i] < 1 || lengths[i] > (1 << 22)) return CPATTN_ERR_INVALID_ARG;
  const int32_t nm = c.m_max - c.m_min + 1;
  if (!out->sample_bucket || !out->bucket_cp || !out->bucket_slot || !out->bucket_rank || !out->bucket_tokens ||
      !out->bucket_load || !out->times || !out->budget ||
      (int64_t)out->bucket_capacity < (int64_t)c.gpus * c.m_max)
    return CPATTN_ERR_INVALID_ARG;

  // std::vector growth inside the planner can throw std::bad_alloc; no
  // exception may cross the C boundary
  try {
    return plan_batch(lengths, n, c, nm, out);
  } catch (...) {
    return CPATTN_ERR_NOMEM;
  }
}

static cpattn_status plan_batch(const int32_t* lengths, int32_t n, const cpattn_dcp_config& c, int32_t nm,
                                cpattn_dcp_plan* out) {
  Planner pl(lengths, n, c);
  // Fig. 7 budget curve and its knee (IEEE double, order as written)
  const double floor_ = (double)pl.wmax() / (double)c.max_cp;
  for (int32_t j = 0; j < nm; ++j) {
    const int32_t mj = c.m_min + j;
    out->budget[j] = std::max((double)pl.total() / (double)((int64_t)c.gpus * mj), floor_);
  }
  int32_t knee = c.m_min;
  if (nm > 1 && out->budget[0] != out->budget[nm - 1]) {
    double best = 0.0;
    for (int32_t j = 0; j < nm; ++j) {
      const double x = (double)j / (double)(nm - 1);
      const double y = (out->budget[j] - out->budget[nm - 1]) / (out->budget[0] - out->budget[nm - 1]);
      const double v = x + y;
      if (j == 0 || v < best) { best = v; knee = c.m_min + j; }
    }
  }
  out->knee = knee;

  Plan best, cur;
  int32_t best_m = -1;
  for (int32_t j = 0; j < nm; ++j) {
    const int32_t mj = c.m_min + j;
    if (c.knee_radius >= 0 && std::abs(mj - knee) > c.knee_radius) { out->times[j] = -2.0; continue; }
    if (!pl.build(mj, cur)) { out->times[j] = -1.0; continue; }
    cur.time = pl.simulate(cur);
    out->times[j] = (double)cur.time / c.max_cp;
    if (best_m < 0 || cur.time < best.time) { std::swap(best, cur); best_m = mj; }
  }
  if (best_m < 0) return CPATTN_ERR_INFEASIBLE;
  out->m = best_m;
  out->num_buckets = (int32_t)best.mbs.size();
  out->step_time = (double)best.time / c.max_cp;
  for (int32_t i = 0; i < n; ++i) out->sample_bucket[i] = best.owner[i];
  for (size_t j = 0; j < best.mbs.size(); ++j) {
    const Mb& mb = best.mbs[j];
    out->bucket_cp[j] = mb.cp;
    out->bucket_slot[j] = mb.slot;
    out->bucket_rank[j] = mb.rank;
    out->bucket_tokens[j] = mb.tokens;
    out->bucket_load[j] = (double)mb.load;
  }
  return CPATTN_OK;
}
