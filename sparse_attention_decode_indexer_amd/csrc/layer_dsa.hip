// The DSA layer after its selection, as one persistent launch, for gfx950: sparse
// attention over the selected rows, the fixed-order split merge and the output projection
// with the residual.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §A DSA layer: from 29 kernels to one: the layer's stages run inside a persistent
//     kernel instead of a chain of launches.
//   §Optimizing inside the kernel: the selected K/V rows are staged on chip split by
//     split; the output-projection weights are fetched before they are needed.
//   §Model Architecture / §Hybrid SWA-DSA Architecture: GQA attention over the selected
//     rows only, sink bias.
//
// One workgroup per compute unit, all resident.  Each workgroup
//   1  requests the W_o rows of its output-projection block (and the residual elements)
//      into registers at once, so they stream in under the attention;
//   2  takes (token, split) attention items in turn: stages the split's 64 selected rows
//      and writes its partial (the code of the standalone attention, attn_core.h);
//   3  takes (token, head, 32-dim slice) merges in turn: combines the token's split
//      partials in split order (the standalone merge's arithmetic);
//   4  reads every token's attention output and computes 16 output columns of
//      x + O . W_o^T, summing sixteen k-partials in the order of the standalone output
//      projection.
// Every arithmetic step is that of the separate kernels, in the same order, so the layer
// output equals the chain of separate launches bit for bit.
//
// Results that cross workgroups (the split partials, the attention output) travel as
// 64-bit words (launch tag << 32 | 32-bit value) written with agent-scope atomic stores;
// the reader polls the words themselves until each carries this launch's tag, so the
// writer never waits for its stores to land and no separate "ready" flag is needed: one
// memory round trip per hand-off.  The tag is the workspace's launch counter + 1 as left
// by the selection that precedes this launch (which advances it once per launch), so it
// differs from the previous layer step's.  Every wait is bounded; a wait that gives up
// sets the workspace's error word.
#include "attn_core.h"
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kOpRows = 16;                     // output columns (W_o rows) per block
constexpr int kOpBlocks = kHidden / kOpRows;    // 256
constexpr int kOpK = kHq * kD;                  // 1024: output-projection reduction length
constexpr int kOpVW = 16;                       // k-partials (the standalone kernel's waves)
constexpr int kOpKw = kOpK / kOpVW;             // 64 per partial
constexpr int kXsS = kOpK + 8;                  // bf16 per attention-output row in LDS
constexpr int kXqS = kOpK + 16;                 // bytes per W8A8 code row in LDS

struct TailParams {
  AttnParams ap;            // attention over the selection (results as tagged words: tpart, tout)
  const uint8_t* w_o;       // [4096][1024] bf16, or e4m3 codes (W8A8)
  const float* w_o_scale;   // [4096] fp32 row scales (W8A8) or nullptr
  const uint16_t* x;        // [T][4096] residual input
  uint16_t* xout;           // [T][4096]
  uint64_t* trace;          // profiling builds: [grid][16] phase timestamps
};

// LDS of the launch
struct TailShared {
  AttnShared<0, kSplitRows> att;
  alignas(16) uint16_t xs[kMaxT][kXsS];         // attention output (bf16)
  alignas(16) uint8_t xq[kMaxT][kXqS];          // W8A8: its e4m3 codes
  float red[kOpVW][16][16];                     // k-partials of the output tile
  float merge[32 * (2 + 32)];                   // merge: one 32-dim slice's partials of every split
  float amax[kMaxT][16];
  float ascale[kMaxT];
  float ainv[kMaxT];
};

// The W_o units of output-projection block b this lane multiplies (k-partials 2w, 2w+1 of
// the sixteen; lane group g = lane >> 4 takes units g, g + 4 of each 64-wide partial).
template <bool F8>
struct WoFrags {
  static constexpr int NU = F8 ? 1 : 2;         // 16-byte units per partial and lane
  Frag8 f[2][NU];
};

template <bool F8>
DSA_DEV void load_wo(const TailParams& tp, int b, WoFrags<F8>& wf) {
  constexpr int ESZ = F8 ? 1 : 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wrow = b * kOpRows + (lane & 15);
#pragma unroll
  for (int vv = 0; vv < 2; ++vv) {
    const int kw0 = (2 * wave + vv) * kOpKw;
    const uint4* wp = reinterpret_cast<const uint4*>(tp.w_o + ((size_t)wrow * kOpK + kw0) * ESZ) + (lane >> 4);
#pragma unroll
    for (int i = 0; i < WoFrags<F8>::NU; ++i) wf.f[vv][i].u = wp[4 * i];
  }
}

// Merged attention output of 32 dims (quarter qtr) of (token t, head h) from its ns split
// partials (tagged words), written as 16 tagged words of two bf16; the arithmetic and order
// of the standalone merge kernel.  The ns x (2 + 32) words (m, l and the slice's values of
// each split) are polled into LDS (thread tid takes words tid, tid + 512, ...), then thread
// d < 32 combines its dim over the splits in split order.  (A whole head per workgroup --
// 4160 words polled by 64 of the workgroups -- took 2.8 us; the chain's merge kernel cuts
// the same work in these 256 slices.)
constexpr int kSliceD = 32;                                                  // dims per merge slice
constexpr int kSliceW = 2 + kSliceD;                                         // words per split
constexpr int kSlicePer = (32 * kSliceW + kSelThreads - 1) / kSelThreads;    // 3 per thread

DSA_DEV void merge_slice(const AttnParams& ap, int t, int h, int qtr, float* vals /* LDS [ns][kSliceW] */,
                         uint32_t tag, uint64_t* trace) {
  (void)trace;
  const int ns = ap.nsplit;
  const int tid = threadIdx.x;
  const int n = ns * kSliceW;
  const int d0 = kSliceD * qtr;
  const uint64_t* pt = ap.tpart + (size_t)t * ns * kHq * kTagPart;
  uint32_t v[kSlicePer];
  poll_words<kSlicePer>([&](int u) {
    int i = tid + u * kSelThreads;
    i = i < n ? i : n - 1;
    const int j = i / kSliceW, w = i - j * kSliceW;
    const int word = w < 2 ? w : tag_dim_word(d0 + (w - 2));
    return pt + ((size_t)j * kHq + h) * kTagPart + word;
  }, tag, v, ap.ctl);
  DSA_MARK(trace, 6);
#pragma unroll
  for (int u = 0; u < kSlicePer; ++u) {
    const int i = tid + u * kSelThreads;
    if (i < n) vals[i] = __uint_as_float(v[u]);
  }
  __syncthreads();
  if (tid < kSliceD) {
    const int d = d0 + tid;
    const float s2 = ap.sink ? ap.sink[h] * 1.4426950408889634f : -__builtin_inff();
    // every split's (m, l, value) read from LDS up front (unrolled), then combined in order
    float mj[32], lj[32], aj[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int jc = j < ns ? j : ns - 1;
      mj[j] = vals[jc * kSliceW];
      lj[j] = vals[jc * kSliceW + 1];
      aj[j] = vals[jc * kSliceW + 2 + tid];
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 32; ++j) M = j < ns ? fmaxf(M, mj[j]) : M;
    M = fmaxf(M, s2);
    float den = 0.0f, o = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (j < ns) {
          const float sc = mj[j] != -__builtin_inff() ? exp2f(mj[j] - M) : 0.0f;
          den = fmaf(lj[j], sc, den);
          o = fmaf(aj[j], sc, o);
        }
      }
      if (s2 != -__builtin_inff()) den += exp2f(s2 - M);
    }
    const float r = den > 0.0f ? o / den : 0.0f;
    // dims d, d + 1 sit in neighbouring lanes: the even lane stores the pair
    const uint32_t b = (uint32_t)f32_to_bf16(r);
    const uint32_t nb = (uint32_t)__shfl_down((int)b, 1, 64);
    if ((d & 1) == 0)
      ast64(ap.tout + (size_t)t * (kOpK / 2) + (h * kD + d) / 2, ((uint64_t)tag << 32) | b | (nb << 16));
  }
  DSA_MARK(trace, 7);
  __syncthreads();
}

}  // namespace

template <bool F8>
__global__ void __launch_bounds__(kSelThreads, 1) dsa_attn_oproj_kernel(TailParams tp) {
  __shared__ TailShared ts;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wg = blockIdx.x;
  const int nwg = gridDim.x;
  const AttnParams& ap = tp.ap;
  const int T = ap.T;
  const int ns = ap.nsplit;
  uint64_t* trace = tp.trace;
  (void)trace;
  DSA_MARK(trace, 0);
  // the launch tag (first needed when an item stores its partial, so the load's latency
  // hides under the item); x_out is not written for a workspace whose error word is set
  const uint64_t ctlw = ald64(reinterpret_cast<const uint64_t*>(ap.ctl + ctl::kEpoch));
  const uint32_t tag = (uint32_t)ctlw + 1u;
  const bool poisoned = (ctlw >> 32) != 0u;
  DSA_MARK(trace, 1);
  // ---- 1) attention items (token, split), round the workgroups; after the first item's
  //      rows are in, this workgroup's first output-projection block (W_o rows, residual,
  //      row scale) is requested: it streams in under the rest, behind the gather
  WoFrags<F8> wf;
  uint16_t xres = 0;
  float wsv = 1.0f;
  int b = wg;
  auto request_wo = [&]() {
    if (b < kOpBlocks) {
      load_wo<F8>(tp, b, wf);
      const int r = tid >> 4, t = tid & 15;
      if (tid < 256 && t < T) xres = tp.x[(size_t)t * kHidden + b * kOpRows + r];
      if (F8) wsv = tp.w_o_scale[b * kOpRows + ((tid >> 4) & 15)];
    }
  };
  bool requested = false;
  for (int i = wg; i < T * ns; i += nwg) {
    attn_split<0, 0, kSplitRows, kSelThreads, true>(ap, i / ns, i % ns, ts.att, nullptr, tag);
    if (!requested) {
      request_wo();
      requested = true;
    }
    __syncthreads();
  }
  if (!requested) request_wo();
  DSA_MARK(trace, 2);
  // ---- 3) (token, head, 32-dim quarter) merges, round the workgroups from the last one
  //      down (the first workgroups are the likeliest to hold a second attention item)
  if (ns > 1) {
    constexpr int QPH = kD / kSliceD;                               // slices per head
    for (int q = nwg - 1 - wg; q < T * kHq * QPH; q += nwg)
      merge_slice(ap, q / (kHq * QPH), (q / QPH) % kHq, q % QPH, ts.merge, tag, trace);
  }
  DSA_MARK(trace, 3);
  // ---- 4) output projection: every token's attention output into LDS (bf16; W8A8: codes):
  //      word tid of each token holds elements 2 tid, 2 tid + 1
  {
    static_assert(kOpK / 2 == kSelThreads, "one output word per thread and token");
    uint32_t o[kMaxT];
    poll_words<kMaxT>([&](int t) { return ap.tout + (size_t)(t < T ? t : T - 1) * (kOpK / 2) + tid; }, tag, o,
                      ap.ctl);
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) *reinterpret_cast<uint32_t*>(&ts.xs[t][2 * tid]) = t < T ? o[t] : 0u;
  }
  __syncthreads();
  DSA_MARK(trace, 4);
  if constexpr (F8) {
    // per-token quantisation: amax over the token's 1024 values, scale and reciprocal, codes
    // of eight elements at a time (the standalone projection's quantiser)
    constexpr int NC = kMaxT * kOpK / 8 / kSelThreads;      // 8-element chunks per thread (2)
    uint32_t y[NC][4];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + u * kSelThreads;
      const int t = c / (kOpK / 8), kk = (c % (kOpK / 8)) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(&ts.xs[t][kk]);
      y[u][0] = v.x; y[u][1] = v.y; y[u][2] = v.z; y[u][3] = v.w;
      const float mx = row16_max(amax_bf16x8(y[u]));
      // token t's chunks are threads 128 t .. 128 t + 127 of round u: two waves, 8 rows
      if ((lane & 15) == 0) ts.amax[t][((c >> 6) & 1) * 4 + (lane >> 4)] = mx;
    }
    __syncthreads();
    if (wave < kMaxT) {
      const float am = wave_max(lane < 8 ? ts.amax[wave][lane] : 0.0f);
      if (lane == 0) {
        ts.ainv[wave] = am > 0.0f ? 448.0f / am : 1.0f;
        ts.ascale[wave] = am > 0.0f ? am / 448.0f : 1.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + u * kSelThreads;
      const int t = c / (kOpK / 8), kk = (c % (kOpK / 8)) * 8;
      *reinterpret_cast<uint2*>(&ts.xq[t][kk]) = e4m3x8_scaled(y[u], ts.ainv[t]);
    }
    __syncthreads();
  }
  for (; b < kOpBlocks; b += nwg) {
    if (b != wg) {
      load_wo<F8>(tp, b, wf);
      const int r = tid >> 4, t = tid & 15;
      if (tid < 256 && t < T) xres = tp.x[(size_t)t * kHidden + b * kOpRows + r];
      if (F8) wsv = tp.w_o_scale[b * kOpRows + ((tid >> 4) & 15)];
    }
    const int tok = lane & 15;
#pragma unroll
    for (int vv = 0; vv < 2; ++vv) {
      const int kw0 = (2 * wave + vv) * kOpKw;
      f32x4_t acc = {};
#pragma unroll
      for (int j = 0; j < WoFrags<F8>::NU; ++j) {
        const int unit = 4 * j + (lane >> 4);
        Frag8 bfr;
        if (F8) bfr.u = *reinterpret_cast<const uint4*>(&ts.xq[tok & 7][kw0 + unit * 16]);
        else bfr.u = *reinterpret_cast<const uint4*>(&ts.xs[tok & 7][kw0 + unit * 8]);
        if (tok >= kMaxT) bfr.u = make_uint4(0u, 0u, 0u, 0u);
        const Frag8 a = wf.f[vv][j];
        if constexpr (F8) {
          const long a0 = (long)(((uint64_t)a.u.y << 32) | a.u.x), a1 = (long)(((uint64_t)a.u.w << 32) | a.u.z);
          const long b0 = (long)(((uint64_t)bfr.u.y << 32) | bfr.u.x), b1 = (long)(((uint64_t)bfr.u.w << 32) | bfr.u.z);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bfr.v, acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ts.red[2 * wave + vv][4 * (lane >> 4) + i][lane & 15] = acc[i];
    }
    __syncthreads();
    if (tid < 256) {
      const int r = tid >> 4, c = tid & 15;
      float v = ts.red[0][r][c];
#pragma unroll
      for (int w = 1; w < kOpVW; ++w) v += ts.red[w][r][c];
      if (F8) v *= ts.ascale[c & 7] * wsv;
      if (c < T && !poisoned) tp.xout[(size_t)c * kHidden + b * kOpRows + r] = f32_to_bf16(v + bf16_to_f32(xres));
    }
    __syncthreads();
  }
  DSA_MARK(trace, 5);
}

size_t layer_tail_tag_bytes(int k) {
  return (size_t)kMaxT * attn_splits(0, k) * kHq * kTagPart * 8 + (size_t)kMaxT * (kOpK / 2) * 8;
}

static void* attn_oproj_fn(bool w8a8) {
  return w8a8 ? (void*)dsa_attn_oproj_kernel<true> : (void*)dsa_attn_oproj_kernel<false>;
}

hipError_t attn_oproj_check_resident(bool w8a8, int num_cu) {
  int64_t cap = 0;
  hipError_t e = resident_capacity(attn_oproj_fn(w8a8), kSelThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  return cap < num_cu ? hipErrorCooperativeLaunchTooLarge : hipSuccess;
}

hipError_t launch_attn_oproj(const int32_t* idx, int T, int64_t L, int k, void* ctlp, const void* q_att,
                             const void* kcache, const void* vcache, float sm_scale, const float* sink, void* tags,
                             const void* w_o, const float* w_o_scale, const void* x, void* xout, int num_cu,
                             hipStream_t st) {
  TailParams tp{};
  AttnParams& ap = tp.ap;
  ap.q = static_cast<const uint16_t*>(q_att);
  ap.kc = static_cast<const uint8_t*>(kcache);
  ap.vc = static_cast<const uint8_t*>(vcache);
  ap.idx = idx;
  ap.k = k;
  ap.T = T;
  ap.L = L;
  ap.sm_log2 = sm_scale * 1.4426950408889634f;
  ap.sink = sink;
  ap.nsplit = attn_splits(0, k);
  uint64_t* tw = static_cast<uint64_t*>(tags);
  ap.tpart = tw;
  ap.tout = tw + (size_t)kMaxT * ap.nsplit * kHq * kTagPart;
  ap.ctl = static_cast<uint32_t*>(ctlp);
  tp.w_o = static_cast<const uint8_t*>(w_o);
  tp.w_o_scale = w_o_scale;
  tp.x = static_cast<const uint16_t*>(x);
  tp.xout = static_cast<uint16_t*>(xout);
#ifdef DSA_TRACE
  tp.trace = dsa_trace_buffer() ? dsa_trace_buffer() + 1024 * 16 : nullptr;   // rows 1024.. of the buffer
#endif
  const bool f8 = w_o_scale != nullptr;
  void* fn = attn_oproj_fn(f8);
  int64_t cap = 0;
  hipError_t e = resident_capacity(fn, kSelThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  if (cap < num_cu) return hipErrorCooperativeLaunchTooLarge;
  void* args[] = {&tp};
  return hipLaunchKernel(fn, dim3(num_cu), dim3(kSelThreads), args, 0, st);
}

}  // namespace dsa
