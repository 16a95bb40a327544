// Sliding-window attention fused with the output projection, for gfx950.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §Hybrid SWA-DSA Architecture: SWA layers attend a 128-token window; GQA with eight
//     query heads per KV head; a sink bias in the softmax.
//   §A DSA layer: from 29 kernels to one: attention and the output projection belong to
//     the same layer step.
//
// The window of an 8-token block spans at most W + T - 1 cache rows, small enough that
// every output-projection workgroup recomputes the whole block's attention on chip
// instead of reading it from a separate attention launch.  This kernel stages the
// window's K and V rows (from the ring, where the projection launch appended the block's
// own rows) and the 64 (token, head) query rows in LDS, requests its 16 rows of W_o right
// after so they stream in under the attention, and runs the steps of swa_core.h.
// Every workgroup computes the same attention output bit for bit (same code, same
// order), so the projection sees one consistent input.
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "swa_core.h"

namespace dsa {

namespace {

using swa::kRowB;
using swa::kRows;

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
  // K rows then Q rows; afterwards the attention output [kMaxT][kXsStride] bf16 and the
  // projection's per-wave partial tiles
  alignas(16) uint8_t kq[kRows * kRowB + swa::kPairs * kRowB];
  alignas(16) uint8_t v[kRows * kRowB];
  alignas(16) float s[swa::kPairs][swa::kSStride];
  float scale[swa::kPairs];
  float tile[16][16];
  alignas(16) float amax[kMaxT][8];
  float ascale[kMaxT];
  float ainv[kMaxT];
};

}  // namespace

template <bool F8>
__global__ void __launch_bounds__(swa::kThreads) swa_out_kernel(SoParams p) {
  __shared__ SoShared sh;
  const swa::Lds l = {sh.kq, sh.v, sh.kq + kRows * kRowB, sh.s, sh.scale, sh.tile, sh.amax, sh.ascale, sh.ainv};
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int T = p.T;
  const int W = p.window;
  DSA_MARK(p.trace, 0);
  swa::WoFrags<F8> wf;                         // the workgroup's W_o rows (requested below)
  float wsv = 1.0f;
  uint16_t xres = 0;                           // residual element of the final add
  float sinkv = 0.0f;                          // sink logit of this thread's softmax row
  // ---- 1) window rows (K, V) and query rows into LDS
  const swa::Window win = swa::window_of(p.pos0, W, T, p.ring_cap);
  {
    uint4 kv[swa::kWinNCH], vv[swa::kWinNCH];
    swa::load_window(tid, p.kc, p.vc, p.ring_cap, win, win.U, kv, vv);
    // query rows: pair = tid >> 4 (token pair >> 3, head pair & 7), chunk tid & 15
    const int pair = tid >> 4, tq = pair >> 3;
    const uint4 qv = *reinterpret_cast<const uint4*>(
        p.q + ((size_t)(tq < T ? tq : T - 1) * kHq + (pair & 7)) * kD + (tid & 15) * 8);
    // the residual element this thread adds at the end and the sink logit of its softmax
    // row are requested now, ahead of W_o, so that neither wait later holds up the other
    {
      const int r = tid >> 4, t = tid & 15;
      if (tid < 256 && t < T) xres = p.x[(size_t)t * kHidden + b * swa::kOutRows + r];
      if (p.sink) sinkv = p.sink[(tid >> 4) & 7];
    }
    // the workgroup's W_o rows (lane & 15 = row, lane >> 4 = k chunk) are requested after
    // the window (needed first); they stream in under the attention
    // W8A8: scale of W_o row (tid >> 4) & 15, the row this thread dequantises in the reduction
    if constexpr (F8) wsv = p.w_o_scale[b * swa::kOutRows + ((tid >> 4) & 15)];
    // every wave's window requests go out before any wave's W_o requests (an execution
    // barrier only), so the CU's memory path returns the window first
    __builtin_amdgcn_s_barrier();
    swa::load_wo<F8>(tid, p.w_o, b, wf);
    swa::store_window(tid, l, kv, vv, 0, 0);
    *reinterpret_cast<uint4*>(l.q + pair * kRowB + (tid & 15) * 16) = tq < T ? qv : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  DSA_MARK(p.trace, 2);
  DSA_MARK_CLK(p.trace, 8);
  // ---- 2-4) attention of the block, 5) its output projection
  swa::attention(tid, l, p.pos0, W, T, p.sm_log2, p.sink != nullptr, sinkv, p.trace);
  DSA_MARK_CLK(p.trace, 9);
  swa::oproj<F8>(tid, l, wf, wsv);
  DSA_MARK(p.trace, 6);
  {
    const int r = tid >> 4, t = tid & 15;
    if (tid < 256 && t < T) {
      const size_t o = (size_t)t * kHidden + b * swa::kOutRows + r;
      p.xout[o] = f32_to_bf16(l.tile[r][t] + bf16_to_f32(xres));
    }
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
  if (w_o_scale) hipLaunchKernelGGL(swa_out_kernel<true>, dim3(kHidden / swa::kOutRows), dim3(swa::kThreads), 0, st, p);
  else hipLaunchKernelGGL(swa_out_kernel<false>, dim3(kHidden / swa::kOutRows), dim3(swa::kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
