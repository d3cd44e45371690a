/* Seeded stress of the library's host-only entry points (index plans, pair
 * counts, the height/width split, the Dynamic-CP planner and their argument
 * checks), built and run under AddressSanitizer by tests/test_host_asan.py:
 * every plan is checked against properties that hold for any input (the
 * ranks' local rows partition the global rows; the ring steps' pair counts
 * add up to the mask's closed form; every sample lands in one microbatch),
 * and the sanitizer checks every host memory access on the way.  No device
 * is touched.  Exits non-zero on the first failed check. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cpattn.h"

#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "check failed, line %d (case %d): %s\n", __LINE__, kase, #cond); \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {                 /* xorshift64* */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}
static int32_t uniform(int32_t lo, int32_t hi) { /* [lo, hi] */
  return lo + (int32_t)(next_u32() % (uint32_t)(hi - lo + 1));
}

static int kase = 0;

/* every global row 0..T-1 appears exactly once among the ranks' local rows */
static int check_cover(const int64_t* l2g_all, int64_t n, int64_t T, unsigned char* seen) {
  int64_t i;
  memset(seen, 0, (size_t)T);
  if (n != T) return 0;
  for (i = 0; i < n; ++i) {
    if (l2g_all[i] < 0 || l2g_all[i] >= T || seen[l2g_all[i]]) return 0;
    seen[l2g_all[i]] = 1;
  }
  return 1;
}

int main(void) {
  enum { MAXSEQ = 9, MAXT = 1 << 16 };
  int32_t cu[MAXSEQ + 1], cu_l[MAXSEQ + 1];
  int64_t* l2g = (int64_t*)malloc(sizeof(int64_t) * MAXT);
  int64_t* all = (int64_t*)malloc(sizeof(int64_t) * MAXT);
  unsigned char* seen = (unsigned char*)malloc(MAXT);
  int i, r, s, n_hw = 0, n_plan = 0;
  if (!l2g || !all || !seen) return 2;

  /* zigzag plans and pair counts */
  for (kase = 0; kase < 300; ++kase) {
    const int32_t cps[5] = {1, 2, 3, 4, 8};
    const int32_t cp = cps[uniform(0, 4)];
    const int32_t nseq = uniform(1, MAXSEQ);
    int64_t T, n = 0, causal = 0, bidir = 0, got_c = 0, got_b = 0;
    cu[0] = 0;
    for (i = 0; i < nseq; ++i) {
      int32_t L = uniform(0, 6000 / nseq);
      L -= L % (2 * cp);
      cu[i + 1] = cu[i] + L;
      causal += (int64_t)L * (L + 1) / 2;
      bidir += (int64_t)L * L;
    }
    T = cu[nseq];
    for (r = 0; r < cp; ++r) {
      CHECK(cpattn_partition_index(cu, nseq, cp, r, cu_l, l2g) == CPATTN_OK);
      CHECK(cu_l[0] == 0 && (int64_t)cu_l[nseq] * cp == T);
      for (i = 0; i < nseq; ++i) CHECK((int64_t)(cu_l[i + 1] - cu_l[i]) * cp == cu[i + 1] - cu[i]);
      memcpy(all + n, l2g, sizeof(int64_t) * (size_t)cu_l[nseq]);
      n += cu_l[nseq];
      for (s = 0; s < cp; ++s) {
        cpattn_step st;
        st.cp = cp;
        st.rank = r;
        st.step = s;
        st.tf_chunk_tokens = 0;
        st.tf_num_chunks = 0;
        got_c += cpattn_count_pairs(cu, nseq, CPATTN_MASK_CAUSAL, &st);
        got_b += cpattn_count_pairs(cu, nseq, CPATTN_MASK_BIDIR, &st);
      }
    }
    CHECK(check_cover(all, n, T, seen));
    CHECK(got_c == causal && got_b == bidir);
    CHECK(cpattn_workspace_size(T / cp, T / cp, nseq) > 0);
  }

  /* balanced teacher-forcing plans */
  for (kase = 300; kase < 420; ++kase) {
    const int32_t cp = uniform(1, 4), B = uniform(1, 90), N = cp * uniform(1, 4), nseq = uniform(1, 3);
    int64_t T, n = 0;
    if ((int64_t)nseq * 2 * B * N > MAXT) continue;
    cu[0] = 0;
    for (i = 0; i < nseq; ++i) cu[i + 1] = cu[i] + 2 * B * N;
    T = cu[nseq];
    for (r = 0; r < cp; ++r) {
      CHECK(cpattn_partition_index_tf(cu, nseq, cp, r, B, N, cu_l, l2g) == CPATTN_OK);
      CHECK((int64_t)cu_l[nseq] * cp == T);
      memcpy(all + n, l2g, sizeof(int64_t) * (size_t)cu_l[nseq]);
      n += cu_l[nseq];
    }
    CHECK(check_cover(all, n, T, seen));
  }

  /* height/width split */
  for (kase = 420; kase < 560; ++kase) {
    const int32_t H = uniform(1, 40), W = uniform(1, 60), F = uniform(1, 4), cp = uniform(1, 8);
    const int32_t nseq = uniform(1, 3);
    int32_t sh = 0, sw = 0;
    int64_t T, n = 0;
    if (cpattn_split_hw(H, W, cp, &sh, &sw) != CPATTN_OK) continue;
    CHECK(sh * sw == cp && H % sh == 0 && W % sw == 0);
    if ((int64_t)nseq * F * H * W > MAXT) continue;
    cu[0] = 0;
    for (i = 0; i < nseq; ++i) cu[i + 1] = cu[i] + F * H * W;
    T = cu[nseq];
    for (r = 0; r < cp; ++r) {
      CHECK(cpattn_partition_index_hw(cu, nseq, F, H, W, sh, sw, r, cu_l, l2g) == CPATTN_OK);
      memcpy(all + n, l2g, sizeof(int64_t) * (size_t)cu_l[nseq]);
      n += cu_l[nseq];
    }
    CHECK(check_cover(all, n, T, seen));
    ++n_hw;
  }

  /* Dynamic-CP planner */
  for (kase = 560; kase < 640; ++kase) {
    cpattn_dcp_config cfg;
    cpattn_dcp_plan p;
    const int32_t n = uniform(1, 400);
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t cap, nm, b;
    cpattn_status st;
    if (!len) return 2;
    memset(&cfg, 0, sizeof(cfg));
    cfg.max_cp = 1 << uniform(0, 3);
    cfg.gpus = cfg.max_cp * uniform(1, 8);
    cfg.pp = uniform(1, 4);
    cfg.vpp = uniform(1, 3);
    cfg.mem_tokens = uniform(1024, 16384);
    cfg.work_quad = uniform(0, 3);
    cfg.work_lin = uniform(1, 200);
    cfg.m_min = uniform(1, 4);
    cfg.m_max = cfg.m_min + uniform(0, 12);
    cfg.knee_radius = uniform(-1, 3);
    for (i = 0; i < n; ++i)   /* mostly samples one rank can hold, a few that need a split */
      len[i] = uniform(1, (int32_t)cfg.mem_tokens * (uniform(0, 9) == 0 ? cfg.max_cp : 1) / 4);
    cap = cfg.gpus * cfg.m_max;
    nm = cfg.m_max - cfg.m_min + 1;
    memset(&p, 0, sizeof(p));
    p.sample_bucket = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    p.bucket_cp = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
    p.bucket_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
    p.bucket_rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
    p.bucket_tokens = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    p.bucket_load = (double*)malloc(sizeof(double) * (size_t)cap);
    p.times = (double*)malloc(sizeof(double) * (size_t)nm);
    p.budget = (double*)malloc(sizeof(double) * (size_t)nm);
    p.bucket_capacity = cap;
    st = cpattn_dcp_plan_batch(len, n, &cfg, &p);
    CHECK(st == CPATTN_OK || st == CPATTN_ERR_INFEASIBLE);
    if (st == CPATTN_OK) {
      ++n_plan;
      int64_t* tok = (int64_t*)calloc((size_t)cap, sizeof(int64_t));
      if (!tok) return 2;
      CHECK(p.m >= cfg.m_min && p.m <= cfg.m_max && p.num_buckets >= 1 && p.num_buckets <= cfg.gpus * p.m);
      for (i = 0; i < n; ++i) {
        CHECK(p.sample_bucket[i] >= 0 && p.sample_bucket[i] < p.num_buckets);
        tok[p.sample_bucket[i]] += len[i];
      }
      for (b = 0; b < p.num_buckets; ++b) {
        CHECK(p.bucket_cp[b] >= 1 && p.bucket_cp[b] <= cfg.max_cp && p.bucket_slot[b] >= 0 && p.bucket_slot[b] < p.m);
        CHECK(p.bucket_rank[b] >= 0 && p.bucket_rank[b] % p.bucket_cp[b] == 0 && p.bucket_rank[b] < cfg.gpus);
        CHECK(tok[b] <= p.bucket_tokens[b] * p.bucket_cp[b]);
        CHECK(p.bucket_tokens[b] <= cfg.mem_tokens);
      }
      free(tok);
    }
    free(len);
    free(p.sample_bucket);
    free(p.bucket_cp);
    free(p.bucket_slot);
    free(p.bucket_rank);
    free(p.bucket_tokens);
    free(p.bucket_load);
    free(p.times);
    free(p.budget);
  }

  /* quotas: every rank finishes together and the quotas add up */
  for (kase = 640; kase < 700; ++kase) {
    int32_t m[16];
    double W[16], total = 0.0, t0 = 0.0;
    const int32_t n = uniform(1, 16), vpp = uniform(1, 4), pp = uniform(1, 8);
    for (i = 0; i < n; ++i) m[i] = uniform(1, 12);
    CHECK(cpattn_dcp_quotas(m, n, vpp, pp, 1000.0, W) == CPATTN_OK);
    for (i = 0; i < n; ++i) {
      const double t = W[i] * (m[i] * vpp + pp - 1);
      total += W[i] * m[i];
      if (i == 0) t0 = t;
      CHECK(t > 0.999999 * t0 && t < 1.000001 * t0);
    }
    CHECK(total > 999.999 && total < 1000.001);
  }

  /* argument checks come back as status codes */
  kase = 700;
  CHECK(cpattn_partition_index(NULL, 1, 2, 0, cu_l, l2g) == CPATTN_ERR_INVALID_ARG);
  cu[0] = 0;
  cu[1] = 6;
  CHECK(cpattn_partition_index(cu, 1, 2, 0, cu_l, l2g) == CPATTN_ERR_INVALID_ARG);   /* 6 % 4 != 0 */
  CHECK(cpattn_partition_index(cu, 1, 2, 2, cu_l, l2g) == CPATTN_ERR_INVALID_ARG);   /* rank >= cp */
  CHECK(cpattn_dcp_quotas(NULL, 1, 1, 1, 1.0, NULL) == CPATTN_ERR_INVALID_ARG);
  CHECK(cpattn_dcp_plan_batch(NULL, 1, NULL, NULL) == CPATTN_ERR_INVALID_ARG);

  free(l2g);
  free(all);
  free(seen);
  if (n_hw < 20 || n_plan < 20) {
    fprintf(stderr, "too few cases exercised: %d height/width splits, %d plans\n", n_hw, n_plan);
    return 1;
  }
  printf("host stress ok (%d height/width splits, %d plans)\n", n_hw, n_plan);
  return 0;
}
