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
// instead of reading it from a separate attention launch:
//   1  the window's K and V rows and the 64 (token, head) query rows are staged in LDS;
//      the workgroup's 16 rows of W_o are requested right after and stream in meanwhile;
//   2  S = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16) in log2e-scaled units;
//   3  softmax per (token, head) in fp32 over the token's window (16 lanes per row,
//      base-2 exponentials, the sink in the denominator); P is written back as bf16
//      hi + lo parts (P = hi + lo to ~2^-16 relative);
//   4  O = P V on the matrix cores (both parts, fp32 accumulation; V read with LDS
//      transpose loads; eight waves), normalised and rounded to bf16 in LDS -- the
//      attention output;
//   5  the output projection of that block plus the residual, as the unfused kernel.
// Every workgroup computes the same attention output bit for bit (same code, same
// order), so the projection sees one consistent input.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kSoThreads = 1024;
constexpr int kSoWaves = kSoThreads / 64;
constexpr int kSoRows = 160;                 // window rows held: W + T - 1 <= 160
constexpr int kSoPairs = kMaxT * kHq;        // 64 (token, head) rows
constexpr int kRowB = kD * 2 + 16;           // padded bf16 row (bytes) of K, V, Q
constexpr int kSStride = 168;                // fp32 per S row; after the softmax: 168 bf16 hi, 168 lo
constexpr int kOutRows = 16;                 // W_o rows (output columns) per workgroup
constexpr int kXsStride = kHq * kD + 8;      // bf16 per attention-output row in LDS

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
  // K rows then Q rows (phases 1-2); afterwards the attention output [kMaxT][kXsStride]
  // bf16 and the projection's per-wave partial tiles
  alignas(16) uint8_t kq[kSoRows * kRowB + kSoPairs * kRowB];
  alignas(16) uint8_t v[kSoRows * kRowB];
  alignas(16) float s[kSoPairs][kSStride];
  float scale[kSoPairs];      // exp2(m - M) / denominator of each (token, head) row
  float tile[16][16];
  alignas(16) float amax[kMaxT][8];  // W8A8: partial maxima of each token's attention output
  float ascale[kMaxT];        // W8A8: activation scale of each token
  float ainv[kMaxT];          // W8A8: 448 / amax of each token (1 for amax = 0)
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Four 16-bit values through the LDS transpose path: within each 16-lane group, lane q
// supplies the 8 bytes at its address and receives element (q & 3) of the values
// supplied by lanes (q >> 2) + 4i, i = 0..3.
DSA_DEV uint2 lds_tr16(const uint8_t* addr) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(reinterpret_cast<uintptr_t>(addr)));
  return __builtin_bit_cast(uint2, r);
}

}  // namespace

template <bool F8>
__global__ void __launch_bounds__(kSoThreads) swa_out_kernel(SoParams p) {
  __shared__ SoShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  const int T = p.T;
  const int W = p.window;
  constexpr int K = kHq * kD;                  // projection reduction length
  constexpr int Kw = K / kSoWaves;             // per wave
  constexpr int NSTEP = Kw / 32;
  constexpr int NU = F8 ? NSTEP / 2 : NSTEP;   // 16-byte weight units per lane group
  constexpr int ESZ = F8 ? 1 : 2;
  constexpr int XQS = K + 16;                  // W8A8: LDS code row stride (bytes)
  static_assert(NU >= 1, "at least one weight unit per lane");
  const int kw0 = wave * Kw;
  DSA_MARK(p.trace, 0);
  Frag8 wf[NU];                                // the workgroup's W_o rows (requested below)
  float wsv = 1.0f;
  uint16_t xres = 0;                           // residual element of the final add
  float sinkv = 0.0f;                          // sink logit of this thread's softmax row
  // ---- 1) window rows: row u holds position pos0 - W + 1 + u, in ring slot
  //      (base + u) mod cap with base = (pos0 - W + 1) mod cap (cap >= W + T - 1 rows)
  const int U = W + T - 1;
  const int64_t first = p.pos0 - W + 1;
  int64_t base = first % p.ring_cap;
  base = base < 0 ? base + p.ring_cap : base;
  {
    constexpr int CH = kSoRows * 16;                          // 16-byte chunks per matrix
    constexpr int NCH = (CH + kSoThreads - 1) / kSoThreads;
    uint4 kv[NCH], vv[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kSoThreads;
      const int row = c >> 4;
      int64_t sl = base + row;
      sl = sl >= p.ring_cap ? sl - p.ring_cap : sl;
      kv[u] = make_uint4(0u, 0u, 0u, 0u);
      vv[u] = kv[u];
      if ((c < CH) & (row < U) & (first + row >= 0)) {   // rows outside the window are not read
        const size_t off = (size_t)sl * (kD * 2) + (c & 15) * 16;
        kv[u] = *reinterpret_cast<const uint4*>(p.kc + off);
        vv[u] = *reinterpret_cast<const uint4*>(p.vc + off);
      }
    }
    // query rows: pair = tid >> 4 (token pair >> 3, head pair & 7), chunk tid & 15
    const int pair = tid >> 4, tq = pair >> 3;
    const uint4 qv = *reinterpret_cast<const uint4*>(
        p.q + ((size_t)(tq < T ? tq : T - 1) * kHq + (pair & 7)) * kD + (tid & 15) * 8);
    // the residual element this thread adds at the end and the sink logit of its softmax
    // row are requested now, ahead of W_o, so that neither wait later holds up the other
    {
      const int r = tid >> 4, t = tid & 15;
      if (tid < 256 && t < T) xres = p.x[(size_t)t * kHidden + b * kOutRows + r];
      if (p.sink) sinkv = p.sink[(tid >> 4) & 7];
    }
    // the workgroup's W_o rows (lane & 15 = row, lane >> 4 = k chunk) are requested after
    // the window (needed first); they stream in under the attention
    // W8A8: scale of W_o row (tid >> 4) & 15, the row this thread dequantises in the reduction
    if constexpr (F8) wsv = p.w_o_scale[b * kOutRows + ((tid >> 4) & 15)];
    // every wave's window requests go out before any wave's W_o requests (an execution
    // barrier only), so the CU's memory path returns the window first
    __builtin_amdgcn_s_barrier();
    const uint4* wp = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.w_o) +
                                                     ((size_t)(b * kOutRows + (lane & 15)) * K + kw0) * ESZ) +
                      (lane >> 4);
#pragma unroll
    for (int i = 0; i < NU; ++i) wf[i].u = wp[4 * i];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kSoThreads;
      if (c < CH) {
        const int o = (c >> 4) * kRowB + (c & 15) * 16;
        *reinterpret_cast<uint4*>(sh.kq + o) = kv[u];
        *reinterpret_cast<uint4*>(sh.v + o) = vv[u];
      }
    }
    *reinterpret_cast<uint4*>(sh.kq + kSoRows * kRowB + pair * kRowB + (tid & 15) * 16) =
        tq < T ? qv : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  DSA_MARK(p.trace, 2);
  // ---- 2) S = K Q^T: wave w < 5 takes rows u = 32 w .. 32 w + 31 against all 64 pairs
  //      (two 32x32 tiles sharing the K operand), K = 128 dims in 8 steps
  if (wave < kSoRows / 32) {
    const uint8_t* ka = sh.kq + (wave * 32 + (lane & 31)) * kRowB + (lane >> 5) * 16;
    const uint8_t* qa = sh.kq + kSoRows * kRowB + (lane & 31) * kRowB + (lane >> 5) * 16;
    f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      Frag8 a, b0, b1;
      a.u = *reinterpret_cast<const uint4*>(ka + ks * 32);
      b0.u = *reinterpret_cast<const uint4*>(qa + ks * 32);
      b1.u = *reinterpret_cast<const uint4*>(qa + 32 * kRowB + ks * 32);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b0.v, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b1.v, acc1, 0, 0, 0);
    }
    // element e of lane l: row u = 32 w + 8 (e >> 2) + 4 (l >> 5) + (e & 3), pair 32 nt + (l & 31)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int u = wave * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      sh.s[lane & 31][u] = acc0[e] * p.sm_log2;
      sh.s[32 + (lane & 31)][u] = acc1[e] * p.sm_log2;
    }
  }
  __syncthreads();
  DSA_MARK(p.trace, 3);
  // ---- 3) softmax of each pair row: 16 lanes, column pairs 2 j + 32 c + {0, 1}.  Token t
  //      sees rows u in [max(t, W - 1 - pos0), min(t + W - 1, U - 1)] (positions
  //      max(0, pos0 + t - W + 1) .. pos0 + t).
  {
    const int pair = tid >> 4, j = tid & 15, t = pair >> 3;
    const int64_t lo64 = (int64_t)(W - 1) - p.pos0;
    const int lo = (int)(lo64 > t ? lo64 : t);
    const int hi = (t + W - 1 < U - 1) ? t + W - 1 : U - 1;
    const uint32_t span = (uint32_t)(hi - lo);                     // u visible <=> u - lo <= span (unsigned)
    constexpr int NC = kSoRows / 32;
    float z[2 * NC];
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int u = 2 * j + 32 * c;
      const float2 v2 = *reinterpret_cast<const float2*>(&sh.s[pair][u]);
      z[2 * c] = (uint32_t)(u - lo) <= span ? v2.x : -__builtin_inff();
      z[2 * c + 1] = (uint32_t)(u + 1 - lo) <= span ? v2.y : -__builtin_inff();
      m = fmaxf(m, fmaxf(z[2 * c], z[2 * c + 1]));
    }
    m = row16_max(m);
    const float ms = m != -__builtin_inff() ? m : 0.0f;    // an empty row: every p = 0
    float l = 0.0f;
    uint32_t* ph = reinterpret_cast<uint32_t*>(&sh.s[pair][0]);     // hi parts: bf16 [0, 168), lo: [168, 336)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float p0 = __builtin_amdgcn_exp2f(z[2 * c] - ms);       // exp2(-inf) = 0
      const float p1 = __builtin_amdgcn_exp2f(z[2 * c + 1] - ms);
      l += p0 + p1;
      const uint32_t h2 = pack_bf16x2(p0, p1);
      const uint32_t l2 = pack_bf16x2(p0 - __uint_as_float(h2 << 16), p1 - __uint_as_float(h2 & 0xffff0000u));
      ph[j + 16 * c] = h2;
      ph[kSStride / 2 + j + 16 * c] = l2;
    }
    l = row16_sum(l);
    if (j == 0) {
      const float sink2 = p.sink ? sinkv * 1.4426950408889634f : -__builtin_inff();
      const float M = fmaxf(m, sink2);
      float sc = 0.0f, den = 0.0f;
      if (M != -__builtin_inff()) {
        if (m != -__builtin_inff()) {
          sc = exp2f(m - M);
          den = l * sc;
        }
        if (sink2 != -__builtin_inff()) den += exp2f(sink2 - M);
      }
      sh.scale[pair] = den > 0.0f ? sc / den : 0.0f;
    }
  }
  __syncthreads();
  DSA_MARK(p.trace, 4);
  // ---- 4) O = P V: wave w < 8 takes pairs 32 (w >> 2) .. +31 and dims 32 (w & 3) .. +31 as
  //      2 tiles of 32 x 32 (tile rows: 16 pairs x {hi, lo} parts; row m -> pair (m & 15),
  //      part m >> 4), K = 160 rows in 10 steps.  Two waves per SIMD hide each other's
  //      operand loads.
  if (wave < 8) {
    const int pb = wave >> 2, db = wave & 3;
    const int m = lane & 31;
    const int poff = ((m >> 4) * kSStride + 8 * (lane >> 5)) * 2;
    const uint8_t* pa0 = reinterpret_cast<const uint8_t*>(&sh.s[pb * 32 + (m & 15)][0]) + poff;
    const uint8_t* pa1 = reinterpret_cast<const uint8_t*>(&sh.s[pb * 32 + 16 + (m & 15)][0]) + poff;
    // transpose-load addresses: 16-lane group g covers dims +16 (g & 1) .. +15 of the tile and
    // rows 8 (g >> 1) .. +7 of the step; lane q of the group points at row (q >> 2), dims
    // 4 (q & 3) .. +3 (then 4 rows further for the second half)
    const int g = lane >> 4, q = lane & 15;
    const uint8_t* vb = sh.v + (8 * (g >> 1) + (q >> 2)) * kRowB + (32 * db + 16 * (g & 1) + 4 * (q & 3)) * 2;
    f32x16_t acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < kSoRows / 16; ++ks) {
      Frag8 a[2], bv;
      a[0].u = *reinterpret_cast<const uint4*>(pa0 + ks * 32);
      a[1].u = *reinterpret_cast<const uint4*>(pa1 + ks * 32);
      const uint2 lo4 = lds_tr16(vb + (16 * ks) * kRowB);
      const uint2 hi4 = lds_tr16(vb + (16 * ks + 4) * kRowB);
      bv.u = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt].v, bv.v, acc[mt], 0, 0, 0);
    }
    // lane l, element e < 8: pair +8 (e >> 2) + 4 (l >> 5) + (e & 3) of the tile (hi part),
    // the same pair's lo part in element e + 8; dim +(l & 31)
    uint16_t* xs = reinterpret_cast<uint16_t*>(sh.kq);
    const int dim = 32 * db + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int pbase = pb * 32 + mt * 16 + 4 * (lane >> 5);
      const float4 s0 = *reinterpret_cast<const float4*>(&sh.scale[pbase]);
      const float4 s1 = *reinterpret_cast<const float4*>(&sh.scale[pbase + 8]);
      const float scl[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pair = pbase + 8 * (e >> 2) + (e & 3);
        xs[(pair >> 3) * kXsStride + (pair & 7) * kD + dim] = f32_to_bf16((acc[mt][e] + acc[mt][e + 8]) * scl[e]);
      }
    }
  }
  __syncthreads();
  DSA_MARK(p.trace, 5);
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(sh.kq);
  uint8_t* xq = sh.v;     // W8A8 codes [kMaxT][XQS] (V is no longer needed)
  if constexpr (F8) {
    // ---- 4b) per-token quantisation of the attention output: thread tid holds elements
    //      8 (tid & 127) .. +7 of token tid >> 7 (two waves per token)
    static_assert(kMaxT * K / 8 == kSoThreads && kMaxT * XQS <= kSoRows * kRowB, "one chunk per thread");
    const int t = tid >> 7, kk = (tid & 127) * 8;
    const uint4 y = *reinterpret_cast<const uint4*>(&xs[t * kXsStride + kk]);
    const uint32_t y4[4] = {y.x, y.y, y.z, y.w};
    const float m = row16_max(amax_bf16x8(y4));
    if ((lane & 15) == 0) sh.amax[t][(wave & 1) * 4 + (lane >> 4)] = m;
    __syncthreads();
    if (wave < kMaxT) {             // wave t folds token t's eight partial maxima
      const float am = wave_max(lane < 8 ? sh.amax[wave][lane] : 0.0f);
      if (lane == 0) {
        sh.ainv[wave] = am > 0.0f ? 448.0f / am : 1.0f;
        sh.ascale[wave] = am > 0.0f ? am / 448.0f : 1.0f;
      }
    }
    __syncthreads();
    *reinterpret_cast<uint2*>(xq + t * XQS + kk) = e4m3x8_scaled(y4, sh.ainv[t]);
    __syncthreads();
  }
  // ---- 5) output projection over this wave's k range, partial tiles summed in wave order
  float (*red)[16][16] = reinterpret_cast<float (*)[16][16]>(sh.kq + kMaxT * kXsStride * 2);
  {
    f32x4_t acc = {};
    const int tok = lane & 15;
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int unit = 4 * j + (lane >> 4);
      Frag8 bfr;
      if (F8) bfr.u = *reinterpret_cast<const uint4*>(xq + (tok & 7) * XQS + kw0 + unit * 16);
      else bfr.u = *reinterpret_cast<const uint4*>(&xs[(tok & 7) * kXsStride + kw0 + unit * 8]);
      if (tok >= kMaxT) bfr.u = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (F8) {
        const Frag8 a = wf[j];
        const long a0 = (long)(((uint64_t)a.u.y << 32) | a.u.x), a1 = (long)(((uint64_t)a.u.w << 32) | a.u.z);
        const long b0 = (long)(((uint64_t)bfr.u.y << 32) | bfr.u.x), b1 = (long)(((uint64_t)bfr.u.w << 32) | bfr.u.z);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j].v, bfr.v, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
  }
  __syncthreads();
  if (tid < 256) {
    const int r = tid >> 4, c = tid & 15;
    float v = red[0][r][c];
#pragma unroll
    for (int w = 1; w < kSoWaves; ++w) v += red[w][r][c];
    if (F8) v *= sh.ascale[c & 7] * wsv;             // W8A8: dequantise (columns >= T unused)
    sh.tile[r][c] = v;
  }
  __syncthreads();
  DSA_MARK(p.trace, 6);
  {
    const int r = tid >> 4, t = tid & 15;
    if (tid < 256 && t < T) {
      const size_t o = (size_t)t * kHidden + b * kOutRows + r;
      p.xout[o] = f32_to_bf16(sh.tile[r][t] + bf16_to_f32(xres));
    }
  }
}

bool swa_out_fits(int T, int window) { return window >= 1 && window + T - 1 <= kSoRows; }

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
  if (w_o_scale) hipLaunchKernelGGL(swa_out_kernel<true>, dim3(kHidden / kOutRows), dim3(kSoThreads), 0, st, p);
  else hipLaunchKernelGGL(swa_out_kernel<false>, dim3(kHidden / kOutRows), dim3(kSoThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
