// Host check of the kernels' mask helpers (context_attention_varlen_amd/csrc/common.h):
//   key_ranges / query_ranges reproduce mask_allowed position by position, and
//   allowed_bits(key_windows(r), pbase, rem) has bit k set exactly when
//   k < rem and in_ranges(r, pbase + k), for the 28 offsets a lane's
//   accumulator block holds,
// over seeded random queries, keys, sequence offsets and teacher-forcing
// shapes.  Built with hipcc (host code only) and run by test_mask_bits.py.
#include <cstdio>
#include <random>

#include "common.h"

using namespace cpattn;

int main() {
  std::mt19937_64 g(20261203);
  long bad = 0, n = 0;
  auto report = [&](const char* what, int mode, long a, long b, long c) {
    if (bad < 8) std::printf("mismatch %s mode %d: %ld %ld %ld\n", what, mode, a, b, c);
    ++bad;
  };
  const int modes[3] = {CPATTN_MASK_CAUSAL, CPATTN_MASK_BIDIR, CPATTN_MASK_TF_BLOCK};
  for (int it = 0; it < 400000; ++it) {
    const int mode = modes[it % 3];
    const int32_t tf_b = 1 + (int32_t)(g() % 80), tf_n = 1 + (int32_t)(g() % 24);
    const int32_t len = mode == CPATTN_MASK_TF_BLOCK ? 2 * tf_b * tf_n : 1 + (int32_t)(g() % 200000);
    const int32_t pq = (int32_t)(g() % len);
    // the interval forms against the position predicate, on keys near pq and at random
    const KeyRanges kr = key_ranges(mode, pq, tf_b, tf_n);
    for (int j = 0; j < 8; ++j) {
      const int64_t near = ((pq + (int64_t)(g() % 9) - 4) % len + len) % len;
      const int32_t pk = j < 4 ? (int32_t)near : (int32_t)(g() % len);
      ++n;
      if (in_ranges(kr, pk) != mask_allowed(mode, pq, pk, tf_b, tf_n)) report("key_ranges", mode, pq, pk, len);
      const KeyRanges qr = query_ranges(mode, pk, tf_b, tf_n);
      if (in_ranges(qr, pq) != mask_allowed(mode, pq, pk, tf_b, tf_n)) report("query_ranges", mode, pq, pk, len);
    }
    // bit sets over a block of 28 offsets starting near the query (diagonal
    // blocks), at chunk edges, or anywhere; rem covers ragged and empty tails
    const int32_t base_choice = (int32_t)(g() % 3);
    int32_t pbase = base_choice == 0 ? pq - (int32_t)(g() % 40) : base_choice == 1 ? (int32_t)((pq / (tf_b ? tf_b : 1)) * tf_b) - 5
                                                                            : (int32_t)(g() % len);
    if (pbase < 0) pbase = 0;
    const int32_t rem = (int32_t)(g() % 50) - 10;
    const KeyRanges rs[2] = {kr, query_ranges(mode, pq, tf_b, tf_n)};
    for (const KeyRanges& r : rs) {
      const unsigned bits = allowed_bits(key_windows(r), pbase, rem);
      for (int k = 0; k < 28; ++k) {
        ++n;
        const bool want = (k < rem) && in_ranges(r, pbase + k);
        if ((((bits >> k) & 1u) != 0u) != want) report("allowed_bits", mode, pbase, k, rem);
      }
    }
  }
  std::printf("%ld mismatches of %ld\n", bad, n);
  if (bad) return 1;
  std::printf("mask bits ok\n");
  return 0;
}
