// A run of consecutive SWA decoder layers as one persistent launch, for gfx950.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §The execution model: stages of the decode loop are fused into larger kernels and
//     the remaining boundaries are bridged on the device, removing launch overhead and
//     host synchronisation between them.
//   §A DSA layer: from 29 kernels to one: input RMSNorm, Q/K/V projections, RoPE,
//     KV-cache writes, attention and the output projection of a layer in one kernel.
//   §Hybrid SWA-DSA Architecture: SWA layers attend a 128-token window (GQA, sink bias).
//
// One workgroup of 1024 threads per compute unit, 256 in all, all resident.  Per layer:
//   P  workgroups 0..159 each project 8 rows of [Q | K | V] (the projection launch's code,
//      proj_core.h): RMSNorm of the layer input, products on the matrix cores, RoPE, the
//      block's K/V rows appended to the ring, and every rounded value published as a
//      tagged word;
//   A  every workgroup requests its window rows (the W - 1 cached positions) and its 16
//      rows of W_o, collects the block's Q/K/V words, computes the whole block's window
//      attention and its 16 output columns plus the residual (the two-launch layer's
//      code, swa_core.h).  The columns leave as tagged words, which the projecting
//      workgroups of the next layer collect as their input (the last layer writes x_out);
//      the next layer's weight rows are requested before the words are awaited, so they
//      stream in meanwhile.
// Every arithmetic step is that of the per-layer launches, in the same order, so the
// result equals one layer step per layer bit for bit.
//
// Measured on MI355X (five SWA layers, 2^20 positions, T = 8): 94 us against 67 us for
// the same layers as back-to-back launches.  The attention and projection phases run as
// fast as in their own launches; the hand-offs do not: each of the 160 projecting
// workgroups pulls the previous layer's whole output (128 KB of tagged words, read past
// the L2 so that every poll sees memory) -- about 7 us per layer against about 2 us for a
// launch boundary, after which the L2 serves the same bytes to every workgroup of an XCD.
// The module step therefore uses this launch only on request.
//
// Hand-offs are 64-bit words (tag << 32 | two bf16) written with agent-scope stores and
// polled by the reader: one memory round trip, no flag, no barrier.  The tag is the
// workspace's launch counter + 1; every workgroup announces with a tagged word of its own
// that it has read the counter, and workgroup 0 advances the counter once all have.
// Waits are bounded: a wait that gives up sets the workspace's error word, after which no
// wait of the launch spins any more, nothing is written to x_out by a workgroup that saw
// the failure, and every later call on the workspace refuses to run.
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "proj_core.h"
#include "swa_core.h"

namespace dsa {

namespace {

constexpr int kChainBlocks = kHidden / swa::kOutRows;             // 256 workgroups
constexpr int kChainProj = kNProjSWA / 8;                          // 160 project 8 rows each
constexpr int kQkvWords = kMaxT * (kNProjSWA / 2);                 // 5120 words per layer
constexpr int kXWords = kMaxT * (kHidden / 2);                     // 16384 words per layer
constexpr int kQkvPer = kQkvWords / swa::kThreads;                 // 5 per thread
constexpr int kNStep = kHidden / kProjWaves / 32;                  // projection k steps per wave
static_assert(kQkvWords % swa::kThreads == 0 && kProjThreads == swa::kThreads, "chain geometry");

// Workspace: [control block][arrival words 256][Q/K/V words per layer][x words per layer but the last]
constexpr size_t kWsArrive = ctl::kBytes;
constexpr size_t kWsQkv = kWsArrive + (size_t)kChainBlocks * sizeof(uint64_t);
constexpr size_t kWsX = kWsQkv + (size_t)kMaxChain * kQkvWords * sizeof(uint64_t);
constexpr size_t kWsEnd = kWsX + (size_t)(kMaxChain - 1) * kXWords * sizeof(uint64_t);

struct ChainLayer {
  const uint16_t* gamma;    // [4096] RMSNorm weights
  const void* w_qkv;        // [1280][4096] bf16
  const void* w_o;          // [4096][1024] bf16
  uint16_t* kring;          // [cap][128] bf16 ring
  uint16_t* vring;
  const float* sink;        // [8] or nullptr
};

struct ChainParams {
  ProjParams pp;            // projection parameters shared by the layers (T, eps, pos0, ring_cap, RoPE)
  ChainLayer layer[kMaxChain];
  int n;                    // layers in this launch
  int window;
  float sm_log2;            // sm_scale * log2(e)
  const uint16_t* x_in;     // [T][4096]
  uint16_t* x_out;          // [T][4096]
  uint32_t* ctl;            // the workspace's control words (launch counter, error word)
  uint64_t* arrive;         // [256] "counter read" words
  uint64_t* qkvw;           // [kMaxChain][5120] Q/K/V words
  uint64_t* xw;             // [kMaxChain - 1][16384] layer-output words
  uint64_t* trace;          // profiling builds: [256][16] phase timestamps
};

// LDS: the projection's, then (after a barrier) the attention's
union ChainShared {
  ProjShared proj;
  struct {
    alignas(16) uint8_t k[swa::kRows * swa::kRowB];
    alignas(16) uint8_t v[swa::kRows * swa::kRowB];
    alignas(16) uint8_t q[swa::kPairs * swa::kRowB];
    alignas(16) float s[swa::kPairs][swa::kSStride];
    float scale[swa::kPairs];
    float tile[16][16];
    alignas(16) float amax[kMaxT][8];
    float ascale[kMaxT];
    float ainv[kMaxT];
    uint16_t xo[kMaxT][swa::kOutRows];   // the workgroup's output columns, paired into words
  } a;
};

}  // namespace

// One layer of the chain (every thread of the workgroup calls it).  xres: the residual
// element of thread (r = tid >> 4, t = tid & 15) < 256, the layer input's column 16 b + r
// of token t, replaced by the layer's output; rot: the rotary factors of a projecting
// thread (formed by the first layer); ok: false once a wait of this thread gave up.
template <bool FIRST>
DSA_DEV void chain_layer(const ChainParams& cp, int li, uint32_t tag, ChainShared& sh, const swa::Lds& l,
                         uint16_t& xres, float2& rot, bool& ok, uint64_t* trace) {
  (void)trace;
  const int T = cp.pp.T;
  const int W = cp.window;
  const swa::Window win = swa::window_of(cp.pp.pos0, W, T, cp.pp.ring_cap);
  const int nw = T * (kNProjSWA / 2);           // Q/K/V words of the block
  if (li == 1) DSA_MARK(trace, 2);
  // the thread and workgroup index are re-read opaquely in every layer, so the compiler
  // does not hoist the phases' index arithmetic out of the loop (its live ranges would
  // spill)
  int tid = threadIdx.x;
  int b = blockIdx.x;
  asm volatile("" : "+v"(tid));
  asm volatile("" : "+s"(b));
  const ChainLayer& L = cp.layer[li];
  uint64_t* const qkvw = cp.qkvw + (size_t)li * kQkvWords;
  // ---- P) projection of 8 rows of [Q | K | V] (workgroups 0..159)
  if (b < kChainProj) {
    const ProjLayer lp{cp.x_in, L.w_qkv, L.gamma, L.kring, L.vring};
    const ProjTags tg{FIRST ? nullptr : cp.xw + (size_t)(li - 1) * kXWords, qkvw, tag, cp.ctl, rot};
    // the first layer reads x_in and forms the rotary factors; the later ones take the
    // layer input from the previous layer's words and reuse the factors (same positions,
    // same rows)
    ok &= proj_body<0, kNStep, true, false, !FIRST, true, !FIRST>(tid, cp.pp, lp, b, sh.proj, tg,
                                                                  li == 1 && trace ? trace + 256 * 16 : nullptr);
    if (FIRST && tid < 8 * kMaxT) rot = make_float2(sh.proj.rc[tid >> 3][tid & 7], sh.proj.rs[tid >> 3][tid & 7]);
  }
  if (li == 1) DSA_MARK(trace, 3);
  // ---- A) window rows of the cached positions, W_o rows, sink; then the block's words
  uint4 kv[swa::kWinNCH], vv[swa::kWinNCH];
  swa::load_window(tid, reinterpret_cast<const uint8_t*>(L.kring), reinterpret_cast<const uint8_t*>(L.vring),
                   cp.pp.ring_cap, win, W - 1, kv, vv);
  const float sinkv = L.sink ? L.sink[(tid >> 4) & 7] : 0.0f;
  swa::WoFrags<false> wf;
  swa::load_wo<false>(tid, L.w_o, b, wf);
  // first one word of each projecting workgroup (its last of the last token), so that
  // waiting costs one load per producer and round; then every word, most already there
  if (tid < kChainProj) {
    uint32_t w1[1];
    ok &= poll_words<1>([&](int) { return qkvw + (size_t)(T - 1) * (kNProjSWA / 2) + tid * 4 + 3; }, tag, w1, cp.ctl);
  }
  __syncthreads();
  uint32_t qv[kQkvPer];
  ok &= poll_words<kQkvPer>([&](int i) {
    const int w = tid + i * swa::kThreads;
    return qkvw + (w < nw ? w : nw - 1);
  }, tag, qv, cp.ctl);
  if (FIRST && b == 0) {
    // every workgroup has read the launch counter once all have announced it: advance it
    uint32_t av[1];
    if (tid < kChainBlocks) ok &= poll_words<1>([&](int) { return cp.arrive + tid; }, tag, av, cp.ctl);
    __syncthreads();
    if (tid == 0) ast(cp.ctl + ctl::kEpoch, tag);
  }
  if (li == 1) DSA_MARK(trace, 4);
  __syncthreads();                            // the projection's LDS is free
  if (li == 1) DSA_MARK(trace, 5);
  swa::store_window(tid, l, kv, vv, W - 1, win.U);
  {
    // query rows of tokens >= T are zero; word w = t * 640 + 4 b' + r carries rows
    // (ra, rb) of projection block b' for token t
    const int pair = tid >> 4;
    if ((pair >> 3) >= T) *reinterpret_cast<uint4*>(l.q + pair * swa::kRowB + (tid & 15) * 16) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kQkvPer; ++i) {
      const int w = tid + i * swa::kThreads;
      if (w < nw) {
        const int t = w / (kNProjSWA / 2), pr = w - t * (kNProjSWA / 2);
        const BlockInfo bi = block_info(pr >> 2, 8);
        const int ra = block_row(bi, pr & 3, 8), rb = block_row(bi, (pr & 3) + 4, 8);
        uint8_t* base;
        int da, db;
        if (ra < kHq * kD) {                  // query head ra >> 7 of token t
          base = l.q + (t * kHq + (ra >> 7)) * swa::kRowB;
          da = ra & (kD - 1);
          db = rb & (kD - 1);
        } else {                              // the block's K or V row of token t
          base = (ra < kHq * kD + kD ? l.k : l.v) + (W - 1 + t) * swa::kRowB;
          const int s0 = ra < kHq * kD + kD ? kHq * kD : kHq * kD + kD;
          da = ra - s0;
          db = rb - s0;
        }
        reinterpret_cast<uint16_t*>(base)[da] = (uint16_t)qv[i];
        reinterpret_cast<uint16_t*>(base)[db] = (uint16_t)(qv[i] >> 16);
      }
    }
  }
  __syncthreads();
  if (li == 1) DSA_MARK(trace, 6);
  swa::attention(tid, l, cp.pp.pos0, W, T, cp.sm_log2, L.sink != nullptr, sinkv,
                 li == 1 && trace ? trace + 512 * 16 : nullptr);
  if (li == 1) DSA_MARK(trace, 7);
  swa::oproj<false>(tid, l, wf, 1.0f);
  // ---- output columns: the last layer writes x_out (unless a wait of this workgroup gave
  //      up), the others publish them as words for the next layer
  const bool last = li == cp.n - 1;
  const bool failed = __syncthreads_or(!ok);
  if (tid < 256) {
    const int r = tid >> 4, t = tid & 15;
    if (t < T) {
      const uint16_t o = f32_to_bf16(l.tile[r][t] + bf16_to_f32(xres));
      xres = o;
      if (last) {
        if (!failed) cp.x_out[(size_t)t * kHidden + b * swa::kOutRows + r] = o;
      } else {
        sh.a.xo[t][r] = o;
      }
    }
  }
  if (!last) {
    __syncthreads();
    if (tid < 8 * T && !failed) {
      const int t = tid >> 3, c2 = tid & 7;
      const uint32_t v = (uint32_t)sh.a.xo[t][2 * c2] | ((uint32_t)sh.a.xo[t][2 * c2 + 1] << 16);
      ast64(cp.xw + (size_t)li * kXWords + (size_t)t * (kHidden / 2) + b * (swa::kOutRows / 2) + c2,
            ((uint64_t)tag << 32) | v);
    }
  }
  if (li == 0) DSA_MARK(trace, 1);
  if (li == 1) DSA_MARK(trace, 8);
}

__global__ void __launch_bounds__(swa::kThreads) swa_chain_kernel(ChainParams cp) {
  __shared__ ChainShared sh;
  const swa::Lds l = {sh.a.k, sh.a.v, sh.a.q, sh.a.s, sh.a.scale, sh.a.tile, sh.a.amax, sh.a.ascale, sh.a.ainv};
  uint64_t* trace = cp.trace;
  // launch counter and error word in one read: a workspace whose earlier launch gave up
  // runs nothing
  const uint64_t ctlw = ald64(reinterpret_cast<const uint64_t*>(cp.ctl + ctl::kEpoch));
  if ((uint32_t)(ctlw >> 32) != 0u) return;
  const uint32_t tag = next_epoch((uint32_t)ctlw);
  if (threadIdx.x == 0) ast64(cp.arrive + blockIdx.x, ((uint64_t)tag << 32) | 1u);
  DSA_MARK(trace, 0);
  uint16_t xres = 0;
  if (threadIdx.x < 256 && (int)(threadIdx.x & 15) < cp.pp.T)
    xres = cp.x_in[(size_t)(threadIdx.x & 15) * kHidden + blockIdx.x * swa::kOutRows + (threadIdx.x >> 4)];
  bool ok = true;
  float2 rot = make_float2(0.0f, 0.0f);
  chain_layer<true>(cp, 0, tag, sh, l, xres, rot, ok, trace);
  for (int li = 1; li < cp.n; ++li) chain_layer<false>(cp, li, tag, sh, l, xres, rot, ok, trace);
}

size_t swa_chain_workspace_bytes() { return kWsEnd; }

bool swa_chain_fits(int T, int window) { return T >= 1 && T <= kMaxT && swa_out_fits(T, window); }

hipError_t swa_chain_check_resident(int num_cu) {
  int64_t cap = 0;
  hipError_t e = resident_capacity(reinterpret_cast<const void*>(&swa_chain_kernel), swa::kThreads, num_cu, &cap);
  if (e != hipSuccess) return e;
  return cap < kChainBlocks ? hipErrorCooperativeLaunchTooLarge : hipSuccess;
}

hipError_t launch_swa_chain(int n, const SwaChainLayer* layers, const void* x_in, void* x_out, int T,
                            int64_t pos0, int window, float sm_scale, float eps, float theta, int64_t ring_cap,
                            void* ws, int num_cu, hipStream_t st) {
  if (n < 1 || n > kMaxChain) return hipErrorInvalidValue;
  if (hipError_t e = swa_chain_check_resident(num_cu)) return e;
  ChainParams cp{};
  ProjParams& p = cp.pp;
  p.T = T;
  p.rpw = 8;
  p.eps = eps;
  p.theta = theta;
  for (int i = 0; i < kD / 2; ++i) p.inv_freq[i] = std::pow((double)theta, -2.0 * (double)i / (double)kD);
  for (int i = 0; i < kDI / 2; ++i) p.inv_freq[kD / 2 + i] = std::pow((double)theta, -2.0 * (double)i / (double)kDI);
  p.pos0 = pos0;
  p.nproj = kNProjSWA;
  p.ring_cap = ring_cap;
  for (int i = 0; i < n; ++i) {
    cp.layer[i].gamma = static_cast<const uint16_t*>(layers[i].gamma);
    cp.layer[i].w_qkv = layers[i].w_qkv;
    cp.layer[i].w_o = layers[i].w_o;
    cp.layer[i].kring = static_cast<uint16_t*>(layers[i].kring);
    cp.layer[i].vring = static_cast<uint16_t*>(layers[i].vring);
    cp.layer[i].sink = layers[i].sink;
  }
  cp.n = n;
  cp.window = window;
  cp.sm_log2 = sm_scale * 1.4426950408889634f;
  cp.x_in = static_cast<const uint16_t*>(x_in);
  cp.x_out = static_cast<uint16_t*>(x_out);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  cp.ctl = reinterpret_cast<uint32_t*>(w8);
  cp.arrive = reinterpret_cast<uint64_t*>(w8 + kWsArrive);
  cp.qkvw = reinterpret_cast<uint64_t*>(w8 + kWsQkv);
  cp.xw = reinterpret_cast<uint64_t*>(w8 + kWsX);
#ifdef DSA_TRACE
  cp.trace = dsa_trace_buffer() ? dsa_trace_buffer() + 1280 * 16 : nullptr;   // rows 1280.. of the buffer
#endif
  hipLaunchKernelGGL(swa_chain_kernel, dim3(kChainBlocks), dim3(swa::kThreads), 0, st, cp);
  return hipGetLastError();
}

}  // namespace dsa
