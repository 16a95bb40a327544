// The DSA layer after its projection, as one launch, for gfx950: indexer scan, exact
// top-k, sparse attention over the selected rows, the fixed-order split merge and the
// output projection with the residual.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §A DSA layer: from 29 kernels to one: the layer's stages run inside one persistent
//     kernel instead of a chain of launches.
//   §Optimizing inside the kernel: the selected K/V rows are staged on chip split by
//     split; the output-projection weights are fetched before they are needed.
//   §Model Architecture / §Hybrid SWA-DSA Architecture: indexer over the full history,
//     top 2,048, GQA attention over the selected rows only, sink bias.
//
// One workgroup per chunk of keys, all resident (as the selection alone).  After the
// selection (select_core.h), each workgroup carries on instead of ending:
//   1  the resolver of token t publishes its indices (agent-scope stores, then a tagged
//      slot) and runs split 0 of token t itself;
//   2  every workgroup requests the W_o rows of its output-projection block (and the
//      residual elements) into registers, long before it needs them;
//   3  the other (token, split) attention items go round the remaining workgroups: each
//      waits for its token's slot, stages its 64 rows and writes its partial (the code of
//      the standalone attention, attn_core.h); the last split of a token to finish (a
//      per-token counter) merges the token's splits in split order and publishes the
//      token's attention output;
//   4  every workgroup waits for all tokens' outputs and computes 16 output columns of
//      x + O . W_o^T, summing sixteen k-partials in the order of the standalone output
//      projection.
// Every arithmetic step is that of the separate kernels, in the same order, so the layer
// output equals the five-launch composition bit for bit.  Cross-workgroup data moves only
// through agent-scope atomic stores/loads and tagged slots; every wait is bounded and a
// wait that gives up sets the workspace's error word.
#include "attn_core.h"
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "select_core.h"

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
  AttnParams ap;            // attention over the selection (ap.out: the bf16 output [T][1024])
  const uint8_t* w_o;       // [4096][1024] bf16, or e4m3 codes (W8A8)
  const float* w_o_scale;   // [4096] fp32 row scales (W8A8) or nullptr
  const uint16_t* x;        // [T][4096] residual input
  uint16_t* xout;           // [T][4096]
  uint32_t* acnt;           // per-token split counters (stride 64 words)
  uint64_t* idxg;           // per-token "indices published" tagged slots (stride 4)
  uint64_t* outg;           // per-token "attention output published" tagged slots (stride 4)
};

// LDS of the phases after the selection (inside the selection's score area)
struct TailShared {
  AttnShared<0, kSplitRows> att;
  alignas(16) uint16_t xs[kMaxT][kXsS];         // attention output (bf16)
  alignas(16) uint8_t xq[kMaxT][kXqS];          // W8A8: its e4m3 codes
  float red[kOpVW][16][16];                     // k-partials of the output tile
  float amax[kMaxT][16];
  float ascale[kMaxT];
  float ainv[kMaxT];
  float2 ml[32 * kHq];                          // merge: (m, l) of every (split, head)
  uint32_t flag;
};

// Wave 0 waits until slots[4 t] carries `tag` for every t < n (bounded), then the block.
DSA_DEV void wait_slots(const uint64_t* slots, int n, uint32_t tag, uint32_t* ctl_words) {
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    const uint64_t* s = slots + 4 * (lane < n ? lane : n - 1);
    uint64_t v = ald64(s);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__ballot((uint32_t)(v >> 32) != tag) != 0ull) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
        if (lane == 0) ast(ctl_words + ctl::kError, 1u);
        break;
      }
      v = ald64(s);
    }
  }
  __syncthreads();
}

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

// Merged attention output of token t (all 1024 elements, two per thread) from its ns
// split partials, written as bf16 with agent-scope stores; the arithmetic and order of
// merge_element (and of the standalone merge kernel).  The splits' (m, l) pairs go
// through LDS (one load per thread); each thread keeps its two elements' 2 x ns values.
DSA_DEV void merge_token(const TailParams& tp, int t, float2* ml_lds) {
  const int ns = tp.ap.nsplit;
  const int tid = threadIdx.x;
  const float* pt = tp.ap.part + (size_t)t * ns * kHq * kPartStride;
  if (tid < ns * kHq) {                              // (split, head) = (tid / 8, tid % 8)
    const uint64_t ml = ald64(reinterpret_cast<const uint64_t*>(pt + (size_t)tid * kPartStride));
    ml_lds[tid] = make_float2(__uint_as_float((uint32_t)ml), __uint_as_float((uint32_t)(ml >> 32)));
  }
  const int e0 = 2 * tid;                            // elements e0, e0 + 1 (same head)
  const int hh = e0 >> 7, d = e0 & (kD - 1);
  float a0[32], a1[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int js = j < ns ? j : ns - 1;
    const uint64_t av = ald64(reinterpret_cast<const uint64_t*>(pt + ((size_t)js * kHq + hh) * kPartStride + 4 + d));
    a0[j] = __uint_as_float((uint32_t)av);
    a1[j] = __uint_as_float((uint32_t)(av >> 32));
  }
  __syncthreads();
  const float s2 = tp.ap.sink ? tp.ap.sink[hh] * 1.4426950408889634f : -__builtin_inff();
  float M = -__builtin_inff();
  for (int j = 0; j < ns; ++j) M = fmaxf(M, ml_lds[j * kHq + hh].x);
  M = fmaxf(M, s2);
  float den = 0.0f, o0 = 0.0f, o1 = 0.0f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j < ns) {
        const float2 ml = ml_lds[j * kHq + hh];
        const float sc = ml.x != -__builtin_inff() ? exp2f(ml.x - M) : 0.0f;
        den = fmaf(ml.y, sc, den);
        o0 = fmaf(a0[j], sc, o0);
        o1 = fmaf(a1[j], sc, o1);
      }
    }
    if (s2 != -__builtin_inff()) den += exp2f(s2 - M);
  }
  const float r0 = den > 0.0f ? o0 / den : 0.0f;
  const float r1 = den > 0.0f ? o1 / den : 0.0f;
  uint16_t* out = static_cast<uint16_t*>(tp.ap.out) + (size_t)t * kOpK + e0;
  ast(reinterpret_cast<uint32_t*>(out), (uint32_t)f32_to_bf16(r0) | ((uint32_t)f32_to_bf16(r1) << 16));
}

}  // namespace

template <int RTW, bool F8>
__global__ void __launch_bounds__(kSelThreads, 1) dsa_layer_tail_kernel(SelParams p, TailParams tp) {
  __shared__ SelShared sh;
  uint32_t epoch;
  if (!select_body<0, 1, RTW, true>(p, sh, epoch)) return;     // poisoned workspace: nothing more
  const uint32_t tag = epoch + 1u;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wg = blockIdx.x;
  const int nwg = p.nwg;
  const int T = p.T;
  const int ns = tp.ap.nsplit;
  TailShared& ts = *reinterpret_cast<TailShared*>(&sh.sc[0][0]);
  static_assert(sizeof(TailShared) <= sizeof(sh.sc), "tail phases fit the score area");

  // ---- 1) resolver: publish token wg's indices (every thread's stores complete first)
  if (wg < T) {
    vm_wait_all();
    __syncthreads();
    if (tid == 0) ast64(tp.idxg + 4 * wg, ((uint64_t)tag << 32) | 1u);
  }
  // ---- 2) this workgroup's first output-projection block: W_o rows, residual, row scale
  WoFrags<F8> wf;
  uint16_t xres = 0;
  float wsv = 1.0f;
  int b = wg;
  if (b < kOpBlocks) {
    load_wo<F8>(tp, b, wf);
    const int r = tid >> 4, t = tid & 15;
    if (tid < 256 && t < T) xres = tp.x[(size_t)t * kHidden + b * kOpRows + r];
    if (F8) wsv = tp.w_o_scale[b * kOpRows + ((tid >> 4) & 15)];
  }
  // ---- 3) attention items: (t, 0) by resolver t, the others round the other workgroups
  const int nrest = T * (ns - 1);
  const int span = nwg > T ? nwg - T : nwg;
  const int first = nwg > T ? wg - T : wg;
  for (int it = (wg < T ? -1 : 0); ; ) {
    int t, s;
    if (it < 0) {
      t = wg;
      s = 0;
    } else {
      const int j = first + it * span;
      if (first < 0 || j >= nrest) break;
      t = j / (ns - 1);
      s = 1 + j % (ns - 1);
    }
    if (!(s == 0 && t == wg)) wait_slots(tp.idxg + 4 * t, 1, tag, p.ctl);
    attn_split<0, 0, kSplitRows, kSelThreads, true>(tp.ap, t, s, ts.att, nullptr);
    vm_wait_all();
    __syncthreads();
    if (ns > 1) {
      if (tid == 0) ts.flag = aadd(tp.acnt + 64 * t, 1u) == (uint32_t)(ns - 1) ? 1u : 0u;
      __syncthreads();
      if (ts.flag) {                  // the last split of token t: merge in split order
        merge_token(tp, t, ts.ml);
        if (tid == 0) ast(tp.acnt + 64 * t, 0u);
        vm_wait_all();
        __syncthreads();
        if (tid == 0) ast64(tp.outg + 4 * t, ((uint64_t)tag << 32) | 1u);
      }
    } else if (tid == 0) {
      ast64(tp.outg + 4 * t, ((uint64_t)tag << 32) | 1u);
    }
    __syncthreads();
    ++it;
  }
  // ---- 4) output projection: every token's attention output into LDS (bf16; W8A8: codes)
  wait_slots(tp.outg, T, tag, p.ctl);
  {
    const uint64_t* src = static_cast<const uint64_t*>(tp.ap.out);
    constexpr int NQ = kMaxT * kOpK / 4 / kSelThreads;     // 64-bit words per thread (4)
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int c = tid + u * kSelThreads;                  // word c: token c / 256, elements 4 (c % 256) ..
      const int t = c / (kOpK / 4), k4 = (c % (kOpK / 4)) * 4;
      const uint64_t v = t < T ? ald64(src + (size_t)t * (kOpK / 4) + k4 / 4) : 0ull;
      *reinterpret_cast<uint64_t*>(&ts.xs[t][k4]) = v;
    }
  }
  __syncthreads();
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
      if (c < T) tp.xout[(size_t)c * kHidden + b * kOpRows + r] = f32_to_bf16(v + bf16_to_f32(xres));
    }
    __syncthreads();
  }
}

hipError_t launch_dsa_layer_tail(const void* q_idx, const float* w_idx, const void* k_idx, const float* k_scale,
                                 int T, int64_t L, int64_t pos0, int k, int32_t* idx, void* ctlp, void* seldata,
                                 const void* q_att, const void* kcache, const void* vcache, float sm_scale,
                                 const float* sink, void* o_buf, void* part, const void* w_o,
                                 const float* w_o_scale, const void* x, void* xout, int num_cu, hipStream_t st) {
  const SelGeometry g = select_geometry(T, L, pos0, k, num_cu);
  SelParams p{};
  p.q_idx = static_cast<const uint16_t*>(q_idx);
  p.w_idx = w_idx;
  p.k_idx = static_cast<const uint8_t*>(k_idx);
  p.k_scale = k_scale;
  p.T = T;
  p.k = k;
  p.L = L;
  p.pos0 = pos0;
  p.chunk = g.chunk;
  p.nwg = g.nwg;
  p.m = g.m;
  p.n_part = g.n_part;
  p.idx = idx;
  p.count = nullptr;
  uint8_t* w8 = static_cast<uint8_t*>(seldata);
  uint32_t* ctl = static_cast<uint32_t*>(ctlp);
  p.ctl = ctl;
  p.cnt = reinterpret_cast<uint64_t*>(w8);
  p.tauv = reinterpret_cast<uint64_t*>(w8 + (size_t)kMaxT * kMaxWG * 8);
  p.cand = reinterpret_cast<uint64_t*>(w8 + (size_t)kMaxT * kMaxWG * 16);
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
  ap.out = o_buf;
  ap.out_f32 = 0;
  ap.part = static_cast<float*>(part);
  ap.nsplit = attn_splits(0, k);
  tp.w_o = static_cast<const uint8_t*>(w_o);
  tp.w_o_scale = w_o_scale;
  tp.x = static_cast<const uint16_t*>(x);
  tp.xout = static_cast<uint16_t*>(xout);
  tp.acnt = ctl + ctl::kAttnCnt;
  tp.idxg = reinterpret_cast<uint64_t*>(ctl + ctl::kIdxG);
  tp.outg = reinterpret_cast<uint64_t*>(ctl + ctl::kOutG);
  const int rt = (T + 1) / 2;
  const bool f8 = w_o_scale != nullptr;
  void* fn = f8 ? (rt == 1 ? (void*)dsa_layer_tail_kernel<1, true> : rt == 2 ? (void*)dsa_layer_tail_kernel<2, true>
                   : rt == 3 ? (void*)dsa_layer_tail_kernel<3, true> : (void*)dsa_layer_tail_kernel<4, true>)
                : (rt == 1 ? (void*)dsa_layer_tail_kernel<1, false> : rt == 2 ? (void*)dsa_layer_tail_kernel<2, false>
                   : rt == 3 ? (void*)dsa_layer_tail_kernel<3, false> : (void*)dsa_layer_tail_kernel<4, false>);
  int64_t cap = 0;
  hipError_t e = resident_capacity(fn, kSelThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  if (cap < g.nwg) return hipErrorCooperativeLaunchTooLarge;
  void* args[] = {&p, &tp};
  return hipLaunchKernel(fn, dim3(g.nwg), dim3(kSelThreads), args, 0, st);
}

hipError_t layer_tail_check_resident(int T, int64_t L, int64_t pos0, int k, bool w8a8, int num_cu) {
  const SelGeometry g = select_geometry(T, L, pos0, k, num_cu);
  const int rt = (T + 1) / 2;
  void* fn = w8a8 ? (rt == 1 ? (void*)dsa_layer_tail_kernel<1, true> : rt == 2 ? (void*)dsa_layer_tail_kernel<2, true>
                     : rt == 3 ? (void*)dsa_layer_tail_kernel<3, true> : (void*)dsa_layer_tail_kernel<4, true>)
                  : (rt == 1 ? (void*)dsa_layer_tail_kernel<1, false> : rt == 2 ? (void*)dsa_layer_tail_kernel<2, false>
                     : rt == 3 ? (void*)dsa_layer_tail_kernel<3, false> : (void*)dsa_layer_tail_kernel<4, false>);
  int64_t cap = 0;
  hipError_t e = resident_capacity(fn, kSelThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  return cap < g.nwg ? hipErrorCooperativeLaunchTooLarge : hipSuccess;
}

}  // namespace dsa
