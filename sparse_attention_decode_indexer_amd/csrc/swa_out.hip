// Sliding-window attention fused with the output projection, for gfx950.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §Hybrid SWA-DSA Architecture: SWA layers attend a 128-token window; GQA with eight
//     query heads per KV head; a sink bias in the softmax.
//   §A DSA layer: from 29 kernels to one: attention and the output projection belong to
//     the same layer step.
//
// The window of an 8-token block spans at most W + T - 1 cache rows, small enough that
// each output-projection workgroup computes the attention it needs on chip instead of
// reading it from a separate attention launch.  Output column n of token t needs only
// token t's attention output, so the 256 workgroups are 2 groups of 4 tokens x 128 blocks
// of 32 output columns (workgroup b = 128 tg + cb: both token groups of a column block
// land on one XCD and share its W_o rows in that XCD's L2).  Each workgroup stages the
// window's K and V rows (from the ring, where the projection launch appended the block's
// own rows) and its group's query rows in LDS, then requests its 32 rows of W_o, which
// stream in under the attention, and runs the token-group steps of swa_core.h: half of
// the whole block's attention.  (One token pair per workgroup halves the attention again,
// but four workgroups then read every W_o row and the L2's bandwidth to the CUs, not the
// attention, sets the time.)  Each value is computed as the whole-block steps compute
// it, so the result does not depend on which workgroup computes it.
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "swa_core.h"

namespace dsa {

namespace {

using swa::kRowB;
using swa::kRows;

constexpr int kG = 4;                               // tokens per workgroup
constexpr int kNGroups = kMaxT / kG;                // 2
constexpr int kCols = 128 / kG;                     // output columns per workgroup (32)
constexpr int kColBlocks = kHidden / kCols;         // 128
constexpr int kNMT = kCols / 16;                    // W_o row tiles per workgroup (2)
constexpr int kGroupPairs = 8 * kG;                 // (token, head) rows of a group (32)
static_assert(kNGroups * kColBlocks == 256 && kCols * kG == 128, "one workgroup per CU; 128 sums per workgroup");

struct SoParams {
  const uint16_t* q;        // [T][8][128] bf16 rotated queries
  const uint8_t* kc;        // ring [cap][128] bf16
  const uint8_t* vc;
  int64_t ring_cap;
  int64_t pos0;
  int T;
  int window;
  float sm_log2;            // sm_scale * log2(e)
  const float* sink;        // [8] natural-log logits or nullptr
  const void* w_o;          // [4096][1024] bf16, or e4m3 codes (W8A8)
  const float* w_o_scale;   // [4096] fp32 row scales (W8A8) or nullptr
  const uint16_t* x;        // [T][4096] residual input
  uint16_t* xout;           // [T][4096]
  uint64_t* trace;          // profiling builds: [blocks][16] phase timestamps
};

struct SoShared {
  // K rows; after the scores the attention output [kMaxT][kXsStride] bf16 and the
  // projection's per-wave partials [16][kCols][kG]
  alignas(16) uint8_t k[kRows * kRowB];
  alignas(16) uint8_t v[kRows * kRowB];              // V rows; then (W8A8) activation codes
  alignas(16) uint8_t q[32 * kRowB];                 // the score tile's 32 query rows
  alignas(16) float s[kGroupPairs][swa::kSStride];
  alignas(16) float scale[kGroupPairs];
  alignas(16) float amax[kMaxT][8];
  float ascale[kMaxT];
  float ainv[kMaxT];
};
static_assert(kMaxT * swa::kXsStride * 2 + 16 * kCols * kG * 4 <= kRows * kRowB, "output and partials fit the K area");

}  // namespace

template <bool F8>
__global__ void __launch_bounds__(swa::kThreads) swa_out_kernel(SoParams p) {
  __shared__ SoShared sh;
  const swa::Lds l = {sh.k, sh.v, sh.q, sh.s, sh.scale, nullptr, sh.amax, sh.ascale, sh.ainv};
  const int tid = threadIdx.x;
  const int tg = blockIdx.x / kColBlocks, cb = blockIdx.x % kColBlocks;
  const int T = p.T;
  const int W = p.window;
  if (kG * tg >= T) return;                          // a token group beyond the block
  DSA_MARK(p.trace, 0);
  uint16_t xres = 0;                                 // residual element of the final add
  float sinkv = 0.0f;                                // sink logit of this thread's softmax row
  float wsv = 1.0f;
  // ---- 1) window rows (K, V) and the group's query rows into LDS
  const swa::Window win = swa::window_of(p.pos0, W, T, p.ring_cap);
  {
    uint4 kv[swa::kWinNCH], vv[swa::kWinNCH];
    swa::load_window(tid, p.kc, p.vc, p.ring_cap, win, win.U, kv, vv);
    // score-tile column c = tid >> 4 < 32 is pair 32 q + c (q = the tile holding the
    // group); the group's columns are loaded, any other column is zero
    const int c = tid >> 4, p0 = kGroupPairs * tg, pair = (p0 & ~31) + c, tq = pair >> 3;
    const bool qreal = tid < 512 && pair >= p0 && pair < p0 + kGroupPairs && tq < T;
    uint4 qv = make_uint4(0u, 0u, 0u, 0u);
    if (qreal) qv = *reinterpret_cast<const uint4*>(p.q + ((size_t)tq * kHq + (pair & 7)) * kD + (tid & 15) * 8);
    // the residual element this thread adds at the end, the sink logit of its softmax row
    // and (W8A8) the scale of the W_o row of its sum
    {
      const int t = kG * tg + (tid % kG);
      if (tid < 128 && t < T) xres = p.x[(size_t)t * kHidden + cb * kCols + tid / kG];
      if (p.sink) sinkv = p.sink[(tid >> 4) & 7];
      if constexpr (F8) if (tid < 128) wsv = p.w_o_scale[cb * kCols + tid / kG];
    }
    swa::store_window(tid, l, kv, vv, 0, 0);
    if (tid < 512) *reinterpret_cast<uint4*>(l.q + c * kRowB + (tid & 15) * 16) = qv;
  }
  __syncthreads();
  // the workgroup's W_o rows are requested once the window is on chip, so the window had
  // the CU's memory path to itself; they stream in under the attention
  swa::WoFrags<F8> wf[kNMT];
#pragma unroll
  for (int mt = 0; mt < kNMT; ++mt) swa::load_wo<F8>(tid, p.w_o, kNMT * cb + mt, wf[mt]);
  DSA_MARK(p.trace, 2);
  DSA_MARK_CLK(p.trace, 8);
  // ---- 2-4) attention of the token group, 5) its output projection
  swa::attention_group<kG>(tid, l, tg, p.pos0, W, T, p.sm_log2, p.sink != nullptr, sinkv, p.trace);
  DSA_MARK_CLK(p.trace, 9);
  const float v = swa::oproj_group<kG, F8>(tid, l, tg, wf, wsv);
  DSA_MARK(p.trace, 6);
  {
    const int t = kG * tg + (tid % kG);
    if (tid < 128 && t < T) p.xout[(size_t)t * kHidden + cb * kCols + tid / kG] = f32_to_bf16(v + bf16_to_f32(xres));
  }
  DSA_MARK(p.trace, 7);
}

bool swa_out_fits(int T, int window) { return window >= 1 && window + T - 1 <= kRows; }

hipError_t launch_swa_out(const void* q, const void* kring, const void* vring, int64_t ring_cap,
                          int64_t pos0, int T, int window, float sm_scale, const float* sink,
                          const void* w_o, const float* w_o_scale, const void* x, void* xout,
                          hipStream_t st) {
  SoParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kc = static_cast<const uint8_t*>(kring);
  p.vc = static_cast<const uint8_t*>(vring);
  p.ring_cap = ring_cap;
  p.pos0 = pos0;
  p.T = T;
  p.window = window;
  p.sm_log2 = sm_scale * 1.4426950408889634f;
  p.sink = sink;
  p.w_o = w_o;
  p.w_o_scale = w_o_scale;
  p.x = static_cast<const uint16_t*>(x);
  p.xout = static_cast<uint16_t*>(xout);
#ifdef DSA_TRACE
  p.trace = dsa_trace_buffer() ? dsa_trace_buffer() + 768 * 16 : nullptr;   // rows 768.. of the buffer
#endif
  if (w_o_scale) hipLaunchKernelGGL(swa_out_kernel<true>, dim3(kNGroups * kColBlocks), dim3(swa::kThreads), 0, st, p);
  else hipLaunchKernelGGL(swa_out_kernel<false>, dim3(kNGroups * kColBlocks), dim3(swa::kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
