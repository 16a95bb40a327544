// Launch geometry of the fused indexer scan + top-k selection (plain C++, no device code,
// so host-side checks can compile it on their own).
//
// The keys [0, L) are cut into chunks of `chunk` keys, one workgroup per chunk and at
// least one workgroup per token (the resolver of token t is workgroup t).  Workgroups
// whose chunk lies wholly before pos0 hold only keys visible to every token; each of
// them publishes a lower bound of its m-th largest score with m * n_part >= min(k, L),
// so at least k scores lie at or above the smallest published bound.
// A chunk of up to kMaxChunk keys keeps its scores for every token in LDS; longer chunks
// (contexts beyond kMaxChunk keys per CU) keep the first kMaxChunk there and the rest in
// the workspace.
// A single token whose whole context is short (T = 1, L <= single_max <= kMaxChunk) takes
// one workgroup that holds every score and selects on chip, without a bound or any
// hand-off.  One CU then streams every key alone, so single_max depends on the bytes per
// key: select_single_max gives it per score source.
#pragma once
#include <stdint.h>

namespace dsa {

constexpr int kSelThreads = 512;   // 8 waves; wave w scores key tiles w, w + 8, ... for all tokens
constexpr int kMaxChunk = 4096;    // keys per workgroup whose scores are held in LDS
constexpr int kMaxSpillChunk = 65536;   // keys per workgroup when the scores past the first
                                        // kMaxChunk of the chunk are kept in the workspace
constexpr int kTauMaxM = 32;       // largest tau rank a workgroup searches (one per lane pair)
constexpr int kMaxWG = 1024;       // slots per token in the count and tau arrays
constexpr int kSelMaxT = 8;        // tokens of a verify block

struct SelGeometry {
  int chunk;    // keys per workgroup (a multiple of kSelThreads)
  int nwg;      // workgroups
  int n_part;   // workgroups [0, n_part) publish a tau bound
  int m;        // tau rank (0: no bound)
  bool fits;    // chunk <= kMaxSpillChunk and nwg fits the count arrays
  bool single;  // one workgroup holds the whole context (T = 1, L <= single_max)
  bool spill;   // chunk > kMaxChunk: scores past the first kMaxChunk keys of each chunk go
                // to the workspace (fused scan) or are read again from the input (loaded
                // scores)
};

// Longest context selected by one workgroup: src 1 = materialised fp32 scores, else the
// indexer keys' storage (kdt 0 = bf16 rows of 128 bytes, 1 = e4m3 rows of 64 bytes plus
// a scale); 0 turns the mode off.  Measured on MI355X (one token, back-to-back calls): one
// workgroup beats the hand-off between workgroups at every length it can hold, for every
// source (bf16 keys at 4096: 21.7 vs 23.7 us; e4m3 at 4096: 12.2 vs 21.9 us).
inline int64_t select_single_max(int src, int kdt) { (void)src; (void)kdt; return kMaxChunk; }

inline SelGeometry select_geometry(int T, int64_t L, int64_t pos0, int k, int num_cu, int64_t single_max) {
  SelGeometry g{};
  if (T == 1 && L >= 1 && L <= single_max && L <= kMaxChunk) {
    g.chunk = (int)((L + kSelThreads - 1) / kSelThreads * kSelThreads);
    g.nwg = 1;
    g.n_part = 0;
    g.m = 0;
    g.fits = true;
    g.single = true;
    return g;
  }
  const int64_t per = (L + num_cu - 1) / num_cu;
  int64_t chunk = ((per + kSelThreads - 1) / kSelThreads) * kSelThreads;
  if (chunk < kSelThreads) chunk = kSelThreads;
  g.chunk = (int)chunk;
  int64_t nwg = (L + chunk - 1) / chunk;
  if (nwg < T) nwg = T;
  g.nwg = (int)nwg;
  g.fits = chunk <= kMaxSpillChunk && nwg <= kMaxWG;
  g.spill = chunk > kMaxChunk;
  g.n_part = (int)(pos0 / chunk);
  const int64_t kmax = (int64_t)k < L ? k : L;
  g.m = 0;
  if (g.n_part >= 1) {
    const int64_t m = (kmax + g.n_part - 1) / g.n_part;
    if (m >= 1 && m <= kTauMaxM) g.m = (int)m;
  }
  return g;
}

// Longest context: one chunk of at most kMaxSpillChunk keys per CU (the workgroups are
// resident one per CU).  Up to kMaxChunk keys per CU every score stays on chip.
inline int64_t select_max_context(int num_cu) { return (int64_t)num_cu * kMaxSpillChunk; }
inline int64_t select_lds_context(int num_cu) { return (int64_t)num_cu * kMaxChunk; }

// candidate slots of a selection workspace sized for (T, L): one chunk per (token,
// workgroup) for the largest block, so any pos0 and T <= kSelMaxT fit (the geometry over
// several workgroups: a single-workgroup launch uses no candidate slots)
inline int64_t select_candidate_slots(int T, int64_t L, int k, int num_cu) {
  const SelGeometry g = select_geometry(T, L, L - T, k, num_cu, 0);
  return (int64_t)kSelMaxT * g.nwg * g.chunk;
}

// spilled scores of a selection workspace sized for (T, L): [kSelMaxT][nwg][chunk -
// kMaxChunk] fp32, only when the chunks exceed kMaxChunk keys
inline int64_t select_spill_floats(int T, int64_t L, int k, int num_cu) {
  const SelGeometry g = select_geometry(T, L, L - T, k, num_cu, 0);
  return g.spill ? (int64_t)kSelMaxT * g.nwg * (g.chunk - kMaxChunk) : 0;
}

}  // namespace dsa
