// Host build of the attention kernels' key/query range helpers: every range
// they return lies in [0, N) with lo <= hi, for valid and invalid
// cu_seqlens tables alike; for valid tables it is the document's range. The
// tile-relative bounds the masks compare in 32 bits select the same
// elements as the 64-bit ranges.
#include <stdio.h>

#include "attn_common.h"

using uly::KeyRange;

static int check(const int32_t *cu, int n_seqs, int64_t N, bool valid) {
  int bad = 0;
  for (int causal = 0; causal < 2; ++causal)
    for (int64_t t = 0; t < N; ++t) {
      const KeyRange k = uly::key_range(cu, n_seqs, N, causal, t);
      const KeyRange q = uly::query_range(cu, n_seqs, N, causal, t);
      for (const KeyRange &r : {k, q})
        if (r.lo < 0 || r.hi > N || r.lo > r.hi) {
          printf("out of range: t=%lld causal=%d [%lld, %lld)\n", (long long)t, causal, (long long)r.lo,
                 (long long)r.hi);
          ++bad;
        }
      // the scanning variants from the document of every earlier token
      for (int64_t t0 = 0; t0 <= t; ++t0) {
        const int b0 = uly::doc_start(cu, n_seqs, t0);
        const KeyRange kf = uly::key_range_from(cu, n_seqs, N, causal, b0, t);
        const KeyRange qf = uly::query_range_from(cu, n_seqs, N, causal, b0, t);
        for (const KeyRange &r : {kf, qf})
          if (r.lo < 0 || r.hi > N || r.lo > r.hi) {
            printf("out of range (scan from %lld): t=%lld causal=%d\n", (long long)t0, (long long)t, causal);
            ++bad;
          }
        if (valid && (kf.lo != k.lo || kf.hi != k.hi || qf.lo != q.lo || qf.hi != q.hi)) {
          printf("scan differs: t0=%lld t=%lld causal=%d\n", (long long)t0, (long long)t, causal);
          ++bad;
        }
      }
      if (valid) {
        int b = 0;
        while (cu[b + 1] <= t) ++b;
        const int64_t lo = cu[b], hi = cu[b + 1];
        if (k.lo != lo || k.hi != (causal ? t + 1 : hi) || q.lo != (causal ? t : lo) || q.hi != hi) {
          printf("wrong range: t=%lld causal=%d\n", (long long)t, causal);
          ++bad;
        }
      }
    }
  return bad;
}

int main() {
  const int32_t good[] = {0, 3, 4, 10, 16};
  const int32_t singles[] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16};  // one token each
  const int32_t past_end[] = {0, 5, 40};          // last document ends past N = 16
  const int32_t negative[] = {-7, 2, 16};
  const int32_t unsorted[] = {0, 12, 5, 16};
  const int32_t huge[] = {0, 2147483647};
  int bad = check(good, 4, 16, true);
  bad += check(singles, 16, 16, true);
  bad += check(past_end, 2, 16, false);
  bad += check(negative, 2, 16, false);
  bad += check(unsorted, 3, 16, false);
  bad += check(huge, 1, 16, false);
  bad += check(nullptr, 0, 16, false);
  // with no table the ranges are the dense ones
  for (int64_t t = 0; t < 16; ++t) {
    const KeyRange k = uly::key_range(nullptr, 0, 16, 1, t), q = uly::query_range(nullptr, 0, 16, 1, t);
    if (k.lo != 0 || k.hi != t + 1 || q.lo != t || q.hi != 16) ++bad;
  }
  // tile-relative 32-bit bounds used for masking: for every element offset
  // E = e + lane_off of a 64-token tile at t0, lo <= t0 + E < hi exactly when
  // rr.lo <= e < rr.hi, also for ranges far outside the tile
  const int64_t far = (int64_t)1 << 40;
  const int64_t ends[] = {-far, -1, 0, 1, 3, 4, 5, 31, 32, 33, 60, 63, 64, 65, 66, 67, 68, 130, far};
  for (const int64_t t0 : {(int64_t)0, (int64_t)64, (int64_t)4096 * 64, far})
    for (const int64_t dl : ends)
      for (const int64_t dh : ends)
        for (int lane_off = 0; lane_off <= 4; lane_off += 4) {
          const int64_t lo = t0 + dl, hi = t0 + dh;
          const uly::RelRange rr = uly::rel_range(lo, hi, t0, lane_off);
          for (int e = 0; e + lane_off < 64; ++e) {
            const int64_t tok = t0 + e + lane_off;
            const bool in_range = tok >= lo && tok < hi, in_rel = e >= rr.lo && e < rr.hi;
            if (in_range != in_rel) {
              printf("rel_range differs: t0=%lld lo=%lld hi=%lld lane_off=%d e=%d\n", (long long)t0, (long long)lo,
                     (long long)hi, lane_off, e);
              ++bad;
            }
          }
        }
  printf("%s\n", bad ? "FAIL" : "OK");
  return bad ? 1 : 0;
}
