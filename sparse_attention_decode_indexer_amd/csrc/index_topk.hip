// Indexer scan and exact top-k selection for gfx950: the materialised-score kernel, the
// selection kernel and their host launchers (device code in select_core.h).
#include <stdlib.h>

#include "dsa_common.h"
#include "dsa_kernels.h"
#include "select_core.h"

namespace dsa {

// ----------------------------------------------------------------------------- scores kernel

constexpr int kScoreThreads = 256;
constexpr int kScoreTilesPerWave = 8;

template <int KDT, int RT>
__global__ void __launch_bounds__(kScoreThreads)
indexer_scores_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                      const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale,
                      int T, int64_t L, int64_t pos0, float* __restrict__ scores, int64_t ld) {
  Frag8 qa[RT][4];
  float wv[RT][16];
  load_q_frags<RT>(q_idx, T, 0, qa);
  load_w<RT>(w_idx, T, 0, wv);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int64_t ntiles = (L + kTile - 1) / kTile;
  const int64_t tile0 = ((int64_t)blockIdx.x * (kScoreThreads / 64) + wave) * kScoreTilesPerWave;
  KeyTile<KDT> buf[kScoreTilesPerWave];
#pragma unroll
  for (int i = 0; i < kScoreTilesPerWave; ++i) {
    const int64_t ti = tile0 + i < ntiles ? tile0 + i : ntiles - 1;
    load_key_tile<KDT>(k_idx, k_scale, L, ti * kTile, buf[i]);
  }
#pragma unroll
  for (int i = 0; i < kScoreTilesPerWave; ++i) {
    const int64_t tile = tile0 + i;
    if (tile >= ntiles) break;
    float out[RT];
    score_tile<KDT, RT>(buf[i], qa, wv, out);
    const int64_t s = tile * kTile + (lane & 31);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int tt = 2 * r + half;
      if (tt < T && s < L) scores[tt * ld + s] = (s <= pos0 + tt) ? out[r] : -__builtin_inff();
    }
  }
}

template <int SRC, int KDT, int RTW, bool SINGLE, bool SPILL = false>
__global__ void __launch_bounds__(kSelThreads, 1) select_kernel(SelParams p) {
  __shared__ SelShared sh;
  uint32_t epoch;
  select_body<SRC, KDT, RTW, SINGLE, SPILL>(p, sh, epoch);
}

// ----------------------------------------------------------------------------- host launchers

static int row_tiles(int T) { return (T + 1) / 2; }

hipError_t launch_indexer_scores(const void* q_idx, const float* w_idx, const void* k_idx,
                                 const float* k_scale, int kdt, int T, int64_t L, int64_t pos0,
                                 float* scores, int64_t ld, hipStream_t st) {
  const int64_t ntiles = (L + kTile - 1) / kTile;
  const int64_t per_block = (kScoreThreads / 64) * kScoreTilesPerWave;
  const dim3 grid((unsigned)((ntiles + per_block - 1) / per_block));
  const dim3 block(kScoreThreads);
  const auto* q = static_cast<const uint16_t*>(q_idx);
  const auto* kk = static_cast<const uint8_t*>(k_idx);
#define DSA_SCORES(KD, RTv) \
  hipLaunchKernelGGL((indexer_scores_kernel<KD, RTv>), grid, block, 0, st, q, w_idx, kk, k_scale, T, L, pos0, scores, ld)
  const int rt = row_tiles(T);
  if (kdt == 0) {
    if (rt == 1) DSA_SCORES(0, 1); else if (rt == 2) DSA_SCORES(0, 2); else if (rt == 3) DSA_SCORES(0, 3); else DSA_SCORES(0, 4);
  } else {
    if (rt == 1) DSA_SCORES(1, 1); else if (rt == 2) DSA_SCORES(1, 2); else if (rt == 3) DSA_SCORES(1, 3); else DSA_SCORES(1, 4);
  }
#undef DSA_SCORES
  return hipGetLastError();
}

// data part of a selection workspace (after the control block): count and tau slots, then
// the candidate lists
size_t select_data_bytes(int T, int64_t L, int k, int num_cu) {
  static_assert(kSelMaxT == kMaxT, "one verify-block limit");
  return (size_t)kMaxT * kMaxWG * (8 + 8) + (size_t)select_candidate_slots(T, L, k, num_cu) * sizeof(uint64_t) +
         (size_t)select_spill_floats(T, L, k, num_cu) * sizeof(float);
}

size_t select_workspace_bytes(int T, int64_t L, int k, int num_cu) {
  return ctl::kBytes + select_data_bytes(T, L, k, num_cu);
}


#ifdef DSA_TRACE
static uint64_t* g_trace = nullptr;
extern "C" void dsa_trace_set(void* buf) { g_trace = static_cast<uint64_t*>(buf); }
uint64_t* dsa_trace_buffer() { return g_trace; }
#endif

static void* select_fn(int src, int kdt, int T, bool single, bool spill) {
  // one token over the whole context in one workgroup
  if (single) return src == 1 ? (void*)select_kernel<1, 0, 1, true>
                    : kdt == 0 ? (void*)select_kernel<0, 0, 1, true> : (void*)select_kernel<0, 1, 1, true>;
  // chunks longer than kMaxChunk keys (scores partly in the workspace): one instance per
  // score source, scoring all four row tiles (rows of absent tokens are zero and unused)
  if (spill) return src == 1 ? (void*)select_kernel<1, 0, 1, false, true>
                   : kdt == 0 ? (void*)select_kernel<0, 0, 4, false, true> : (void*)select_kernel<0, 1, 4, false, true>;
  // every wave scores all ceil(T/2) row tiles of its key tiles
  const int rt = row_tiles(T);
  if (src == 1) return (void*)select_kernel<1, 0, 1, false>;
  if (kdt == 0)
    return rt == 1 ? (void*)select_kernel<0, 0, 1, false> : rt == 2 ? (void*)select_kernel<0, 0, 2, false>
         : rt == 3 ? (void*)select_kernel<0, 0, 3, false> : (void*)select_kernel<0, 0, 4, false>;
  return rt == 1 ? (void*)select_kernel<0, 1, 1, false> : rt == 2 ? (void*)select_kernel<0, 1, 2, false>
       : rt == 3 ? (void*)select_kernel<0, 1, 3, false> : (void*)select_kernel<0, 1, 4, false>;
}

// Workgroups `fn` can hold resident at once on the device (blocks per CU x CUs).  Test
// hook: the environment variable DSA_RESIDENT_LIMIT, when set to a positive number, caps
// the result, standing in for CUs held by other work.
// (The CU count is the device's own: a smaller num_cu only shapes the launch geometry.)
hipError_t resident_capacity(const void* fn, int threads, int num_cu, int64_t* cap) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0);
  if (e != hipSuccess) return e;
  int dev = 0, ncu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  int64_t c = (int64_t)per_cu * (ncu > num_cu ? ncu : num_cu);
  if (const char* lim = getenv("DSA_RESIDENT_LIMIT")) {
    const long v = strtol(lim, nullptr, 10);
    if (v > 0 && v < c) c = v;
  }
  *cap = c;
  return hipSuccess;
}

hipError_t select_check_resident(int src, int kdt, int T, int64_t L, int64_t pos0, int k, int num_cu) {
  const SelGeometry g = select_geometry(T, L, pos0, k, num_cu, select_single_max(src, kdt));
  int64_t cap = 0;
  hipError_t e = resident_capacity(select_fn(src, kdt, T, g.single, g.spill), kSelThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  return cap < g.nwg ? hipErrorCooperativeLaunchTooLarge : hipSuccess;
}

hipError_t launch_select(int src, const void* q_idx, const float* w_idx, const void* k_idx,
                         const float* k_scale, int kdt, const float* scores, int64_t ld, int T,
                         int64_t L, int64_t pos0, int k, int32_t* idx, int32_t* count, void* ctlp,
                         void* data, int num_cu, hipStream_t st) {
  SelGeometry g = select_geometry(T, L, pos0, k, num_cu, select_single_max(src, kdt));
  SelParams p{};
  p.q_idx = static_cast<const uint16_t*>(q_idx);
  p.w_idx = w_idx;
  p.k_idx = static_cast<const uint8_t*>(k_idx);
  p.k_scale = k_scale;
  p.scores = scores;
  p.ld = ld;
  p.T = T;
  p.k = k;
  p.L = L;
  p.pos0 = pos0;
  p.chunk = g.chunk;
  p.nwg = g.nwg;
  p.m = g.m;
  p.n_part = g.n_part;
  p.idx = idx;
  p.count = count;
#ifdef DSA_TRACE
  p.trace = g_trace;
#endif
  uint8_t* w8 = static_cast<uint8_t*>(data);
  p.ctl = static_cast<uint32_t*>(ctlp);
  p.cnt = reinterpret_cast<uint64_t*>(w8);
  p.tauv = reinterpret_cast<uint64_t*>(w8 + (size_t)kMaxT * kMaxWG * 8);
  p.cand = reinterpret_cast<uint64_t*>(w8 + (size_t)kMaxT * kMaxWG * 16);
  // spill rows after this launch's candidate slots (the workspace holds at least that many)
  p.sstride = g.spill ? (int64_t)g.nwg * (g.chunk - kMaxChunk) : 0;
  p.spill = g.spill ? reinterpret_cast<float*>(p.cand + (size_t)kSelMaxT * g.nwg * g.chunk) : nullptr;
  void* args[] = {&p};
  void* fn = select_fn(src, kdt, T, g.single, g.spill);
  // every workgroup must be resident at once (one per CU by the LDS footprint)
  int64_t cap = 0;
  hipError_t e = resident_capacity(fn, kSelThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  if (cap < g.nwg) return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel(fn, dim3(g.nwg), dim3(kSelThreads), args, 0, st);
}

}  // namespace dsa
