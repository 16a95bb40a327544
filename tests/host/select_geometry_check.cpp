// Host-side check of the selection's launch geometry (select_geometry.h): for every
// workgroup, the score rows the materialised path reads, the key rows the fused scan
// reads and the candidate slots it writes stay inside their buffers, and the tau bound
// is valid.  The read ranges restate the kernel's own index expressions.
#include <stdio.h>
#include <stdint.h>

#include <initializer_list>

#include "select_geometry.h"

using namespace dsa;

static int fails = 0;
static long cases = 0;

#define CHECK(c, ...)                                                        \
  do {                                                                       \
    if (!(c)) {                                                              \
      if (fails++ < 20) { printf("FAIL %s: ", #c); printf(__VA_ARGS__); printf("\n"); } \
    }                                                                        \
  } while (0)

static void check(int T, int64_t L, int64_t pos0, int k, int ncu, int64_t single_max) {
  ++cases;
  const SelGeometry g = select_geometry(T, L, pos0, k, ncu, single_max);
  const SelGeometry gw = select_geometry(T, L, L - T, k, ncu, single_max);   // the same block at its last position
  const int64_t ld = (L + 3) / 4 * 4;
  CHECK(g.chunk % kSelThreads == 0 && g.chunk >= kSelThreads, "T=%d L=%lld chunk=%d", T, (long long)L, g.chunk);
  CHECK((int64_t)g.nwg * g.chunk >= L && g.nwg >= T, "T=%d L=%lld nwg=%d", T, (long long)L, g.nwg);
  CHECK(g.chunk == gw.chunk && g.nwg == gw.nwg, "geometry depends on pos0: T=%d L=%lld", T, (long long)L);
  if (L <= select_max_context(ncu)) CHECK(g.fits, "T=%d L=%lld ncu=%d does not fit", T, (long long)L, ncu);
  // one workgroup holding the whole context exactly when T = 1 and L <= single_max (and
  // one chunk): its scores, candidates and histogram stay in LDS (static_asserts there)
  CHECK(g.single == (T == 1 && L <= single_max && L <= kMaxChunk), "single T=%d L=%lld", T, (long long)L);
  if (g.single) CHECK(g.nwg == 1 && g.m == 0 && g.chunk >= L && g.chunk <= kMaxChunk, "single geometry L=%lld", (long long)L);
  // tau: participating chunks lie wholly before pos0 and together hold >= min(k, L) bounds
  if (g.m > 0) {
    const int64_t kmax = k < L ? k : L;
    CHECK((int64_t)g.m * g.n_part >= kmax && (int64_t)g.n_part * g.chunk <= pos0, "tau T=%d L=%lld pos0=%lld k=%d",
          T, (long long)L, (long long)pos0, k);
  }
  const int64_t cand_slots = select_candidate_slots(T, L, k, ncu);   // the workspace's candidate capacity
  const int64_t spill_cap = select_spill_floats(T, L, k, ncu);       // and spill capacity
  CHECK(g.spill == (g.chunk > kMaxChunk) && (g.spill ? spill_cap > 0 : spill_cap == 0), "spill T=%d L=%lld", T,
        (long long)L);
  // row offsets of the spill rows (r * 2 * sstride, r < 4) and candidate offsets stay in 32 bits
  CHECK(7 * (int64_t)g.nwg * g.chunk < ((int64_t)1 << 31), "offsets T=%d L=%lld", T, (long long)L);
  for (int wg = 0; wg < g.nwg; ++wg) {
    const int64_t c0 = (int64_t)wg * g.chunk;
    int64_t nk64 = L - c0;
    nk64 = nk64 < 0 ? 0 : (nk64 > g.chunk ? g.chunk : nk64);
    const int nkeys = (int)nk64;
    for (int t = 0; t < T; ++t) {
      // materialised scores: a workgroup with keys reads src[i < nkeys ? i : nkeys - 1],
      // i < kMaxChunk, from row t at column c0; one without keys reads nothing
      if (nkeys > 0) {
        const int64_t lo = t * ld + c0, hi = t * ld + c0 + (kMaxChunk - 1 < nkeys - 1 ? kMaxChunk - 1 : nkeys - 1);
        CHECK(lo >= t * ld && hi < t * ld + L, "scores T=%d L=%lld wg=%d t=%d [%lld, %lld]", T, (long long)L, wg, t,
              (long long)lo, (long long)hi);
      }
      // candidate slots of (t, wg): at most nkeys written from (t * nwg + wg) * chunk
      const int64_t end = ((int64_t)t * g.nwg + wg) * g.chunk + nkeys;
      CHECK(end <= cand_slots, "candidates T=%d L=%lld wg=%d t=%d", T, (long long)L, wg, t);
    }
    // chunks longer than kMaxChunk: the fused scan writes local positions [kMaxChunk,
    // roundup32(nkeys)) of all kSelMaxT token rows (four row tiles) to the spill rows at
    // t * sstride + wg * (chunk - kMaxChunk) + (pos - kMaxChunk); the candidate pass reads,
    // per kMaxChunk positions from sb, whole float4s up to the last visible position; the
    // loaded-score source reads those from its own row t instead
    if (g.spill && nkeys > kMaxChunk) {
      const int64_t sstride = (int64_t)g.nwg * (g.chunk - kMaxChunk);
      const int64_t seg = (int64_t)wg * (g.chunk - kMaxChunk);
      const int64_t wr_hi = (nkeys + 31) / 32 * 32;
      CHECK(wr_hi <= g.chunk, "spill rows T=%d L=%lld wg=%d", T, (long long)L, wg);
      CHECK((kSelMaxT - 1) * sstride + seg + (wr_hi - 1 - kMaxChunk) < spill_cap, "spill writes T=%d L=%lld wg=%d",
            T, (long long)L, wg);
      for (int t = 0; t < T; ++t) {
        int64_t lim = pos0 + t - c0;
        lim = lim < nkeys - 1 ? lim : nkeys - 1;
        for (int64_t sb = kMaxChunk; sb < nkeys; sb += kMaxChunk) {
          const int64_t nvis = lim - sb + 1;
          if (nvis <= 0) continue;
          const int64_t rd = (nvis + 3) / 4 * 4;          // float4s starting before the last visible one
          CHECK(sb - kMaxChunk + rd <= g.chunk - kMaxChunk && t * sstride + seg + (sb - kMaxChunk) + rd <= spill_cap,
                "spill reads T=%d L=%lld wg=%d t=%d sb=%lld", T, (long long)L, wg, t, (long long)sb);
          CHECK(c0 + sb + rd <= ld, "score row reads T=%d L=%lld wg=%d t=%d", T, (long long)L, wg, t);
        }
      }
    }
    // fused scan: wave w's tiles start at c0 + 32 (w + 8 j), rows past L clamped to L - 1
    const int ntiles = (nkeys + 31) / 32;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      const int nmine = ntiles > w ? (ntiles - w + 7) / 8 : 0;
      const int jlast = nmine > 0 ? nmine - 1 : 0;
      for (int j = 0; j <= jlast + 2; ++j) {          // the prefetch runs two tiles past the last
        const int jc = j < jlast ? j : jlast;
        int64_t s0 = c0 + (int64_t)(w + jc * 8) * 32;
        for (int l = 0; l < 32; l += 31) {
          int64_t s = s0 + l;
          s = s < L ? s : L - 1;
          CHECK(s >= 0 && s < L, "keys T=%d L=%lld wg=%d", T, (long long)L, wg);
        }
      }
    }
  }
}

int main() {
  const int ks[] = {1, 4, 7, 64, 100, 1000, 2048};
  for (int ncu : {256, 80, 32, 1}) {
    for (int64_t L = 1; L <= 6000; L += (L < 600 ? 1 : 37)) {
      for (int T = 1; T <= 8; ++T) {
        if (T > L) continue;
        for (int k : ks) {
          const int64_t p[3] = {L - T, 0, (L - T) / 2};
          for (int64_t pos0 : p)
            for (int64_t sm : {(int64_t)0, select_single_max(0, 0), select_single_max(0, 1), select_single_max(1, 0)})
              check(T, L, pos0, k, ncu, sm);
        }
      }
    }
    for (int64_t L : {(int64_t)65536, (int64_t)262144, (int64_t)1048576, (int64_t)ncu * kMaxChunk,
                      (int64_t)ncu * kMaxChunk - 1, (int64_t)ncu * kMaxChunk + 1, (int64_t)ncu * kMaxChunk + 777,
                      (int64_t)ncu * 3 * kMaxChunk - 5, (int64_t)ncu * kMaxSpillChunk - 1,
                      (int64_t)ncu * kMaxSpillChunk})
      for (int T : {1, 7, 8})
        for (int k : {1, 2048}) {
          check(T, L, L - T, k, ncu, select_single_max(0, 1));
          check(T, L, (L - T) / 3, k, ncu, select_single_max(0, 1));
        }
    // one past the longest context no longer fits
    const SelGeometry gx = select_geometry(8, select_max_context(ncu) + 512, select_max_context(ncu) - 8 + 512, 2048,
                                           ncu, 0);
    CHECK(!gx.fits, "ncu=%d: a context past the limit fits", ncu);
  }
  // the long-chunk shapes the GPU tests run with the geometry cut for a few CUs
  for (int ncu : {1, 2, 3, 4})
    for (int64_t L : {(int64_t)4097, (int64_t)8193, (int64_t)12345, (int64_t)20000, (int64_t)25000, (int64_t)30000,
                      (int64_t)33333, (int64_t)40000, (int64_t)50000, (int64_t)50001, (int64_t)65536, (int64_t)70000,
                      (int64_t)131072})
      for (int T = 1; T <= 8; ++T)
        for (int k : {1000, 2048})
          for (int64_t pos0 : {L - T, L / 2, L / 3})
            if (L <= select_max_context(ncu)) check(T, L, pos0, k, ncu, select_single_max(0, 1));
  printf("%s: %ld cases, %d failures\n", fails ? "FAILED" : "ok", cases, fails);
  return fails ? 1 : 0;
}
