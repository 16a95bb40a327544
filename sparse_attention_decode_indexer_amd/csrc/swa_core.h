// Device code of the sliding-window attention of one block and its output projection,
// for gfx950: shared by the two-launch SWA layer (swa_out_kernel after the projection
// launch) and the persistent multi-layer SWA kernel, so both compute the same bits.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §Hybrid SWA-DSA Architecture: SWA layers attend a 128-token window; GQA with eight
//     query heads per KV head; a sink bias in the softmax.
//   §A DSA layer: from 29 kernels to one: attention and the output projection belong to
//     the same layer step.
//
// The window of a block of T <= 8 tokens spans W + T - 1 <= 160 cache rows, small enough
// for one workgroup of 1024 threads to compute the whole block's attention on chip:
//   1  the window's K and V rows and the 64 (token, head) query rows sit in LDS;
//   2  S = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16) in log2e-scaled units;
//   3  softmax per (token, head) in fp32 over the token's window (16 lanes per row,
//      base-2 exponentials, the sink in the denominator); P is written back as bf16
//      hi + lo parts (P = hi + lo to ~2^-16 relative);
//   4  O = P V on the matrix cores (both parts, fp32 accumulation; V read with LDS
//      transpose loads; eight waves), normalised and rounded to bf16 in LDS -- the
//      attention output;
//   5  16 output columns of O . W_o^T, sixteen k-partials summed in wave order.
#pragma once
#include "dsa_common.h"

namespace dsa {
namespace swa {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 160;                  // window rows held: W + T - 1 <= 160
constexpr int kPairs = kMaxT * kHq;         // 64 (token, head) rows
constexpr int kRowB = kD * 2 + 16;          // padded bf16 row (bytes) of K, V, Q
constexpr int kSStride = 168;               // fp32 per S row; after the softmax: 168 bf16 hi, 168 lo
constexpr int kOutRows = 16;                // W_o rows (output columns) per workgroup
constexpr int kXsStride = kHq * kD + 8;     // bf16 per attention-output row in LDS
constexpr int kOK = kHq * kD;               // output-projection reduction length (1024)
constexpr int kWinCh = kRows * 16;          // 16-byte chunks per window matrix
constexpr int kWinNCH = (kWinCh + kThreads - 1) / kThreads;

// LDS of one block's window attention (pointers into the caller's shared memory)
struct Lds {
  uint8_t* k;                 // [kRows][kRowB] K rows; after the scores: the attention output
                              // [kMaxT][kXsStride] bf16, then the sixteen partial tiles
  uint8_t* v;                 // [kRows][kRowB] V rows; after P.V (W8A8): activation codes
  uint8_t* q;                 // [kPairs][kRowB] query rows, pair = token * 8 + head
  float (*s)[kSStride];       // [kPairs] scores; after the softmax bf16 hi / lo parts of P
  float* scale;               // [kPairs] exp2(m - M) / denominator of each pair row
  float (*tile)[16];          // [16][16] output tile (W_o row, token)
  float (*amax)[8];           // W8A8 [kMaxT][8] partial maxima of the attention output
  float* ascale;              // W8A8 [kMaxT] activation scale of each token
  float* ainv;                // W8A8 [kMaxT] 448 / amax of each token (1 for amax = 0)
};

// Window of the block: row u holds position first + u, in ring slot (base + u) mod cap
// (cap >= W + T - 1 rows); rows at negative positions are outside the context.
struct Window {
  int64_t first;
  int64_t base;
  int U;                      // rows W + T - 1
};

DSA_DEV Window window_of(int64_t pos0, int W, int T, int64_t cap) {
  Window w;
  w.U = W + T - 1;
  w.first = pos0 - W + 1;
  int64_t base = w.first % cap;
  w.base = base < 0 ? base + cap : base;
  return w;
}

// Requests window rows u < u_end (the others, and rows before position 0, read as zero):
// chunk c = tid + 1024 i covers bytes 16 (c & 15) .. +15 of row c >> 4.
DSA_DEV void load_window(int tid, const uint8_t* kc, const uint8_t* vc, int64_t cap, const Window& w, int u_end,
                         uint4 (&kv)[kWinNCH], uint4 (&vv)[kWinNCH]) {
#pragma unroll
  for (int u = 0; u < kWinNCH; ++u) {
    const int c = tid + u * kThreads;
    const int row = c >> 4;
    int64_t sl = w.base + row;
    sl = sl >= cap ? sl - cap : sl;
    kv[u] = make_uint4(0u, 0u, 0u, 0u);
    vv[u] = kv[u];
    if ((c < kWinCh) & (row < u_end) & (w.first + row >= 0)) {   // rows outside the window are not read
      const size_t off = (size_t)sl * (kD * 2) + (c & 15) * 16;
      kv[u] = *reinterpret_cast<const uint4*>(kc + off);
      vv[u] = *reinterpret_cast<const uint4*>(vc + off);
    }
  }
}

// Rows in [skip_lo, skip_hi) are left to the caller.
DSA_DEV void store_window(int tid, const Lds& l, const uint4 (&kv)[kWinNCH], const uint4 (&vv)[kWinNCH],
                          int skip_lo, int skip_hi) {
#pragma unroll
  for (int u = 0; u < kWinNCH; ++u) {
    const int c = tid + u * kThreads;
    if (c < kWinCh && !((c >> 4) >= skip_lo && (c >> 4) < skip_hi)) {
      const int o = (c >> 4) * kRowB + (c & 15) * 16;
      *reinterpret_cast<uint4*>(l.k + o) = kv[u];
      *reinterpret_cast<uint4*>(l.v + o) = vv[u];
    }
  }
}


// The functions take the thread's index as an argument (a caller running them in a loop
// can keep the compiler from hoisting index arithmetic out of it).
//
// Steps 2-4 with K, V and Q in LDS (every thread calls; synchronises internally and at the
// end).  sinkv: the sink logit of head (tid >> 4) & 7 when sink is set.
DSA_DEV void attention(int tid, const Lds& l, int64_t pos0, int W, int T, float sm_log2, bool has_sink, float sinkv,
                       uint64_t* trace) {
  (void)trace;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int U = W + T - 1;
  // ---- 2) S = K Q^T: wave w < 5 takes rows u = 32 w .. 32 w + 31 against all 64 pairs
  //      (two 32x32 tiles sharing the K operand), K = 128 dims in 8 steps
  if (wave < kRows / 32) {
    const uint8_t* ka = l.k + (wave * 32 + (lane & 31)) * kRowB + (lane >> 5) * 16;
    const uint8_t* qa = l.q + (lane & 31) * kRowB + (lane >> 5) * 16;
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
      l.s[lane & 31][u] = acc0[e] * sm_log2;
      l.s[32 + (lane & 31)][u] = acc1[e] * sm_log2;
    }
  }
  __syncthreads();
  DSA_MARK(trace, 3);
  // ---- 3) softmax of each pair row: 16 lanes, column pairs 2 j + 32 c + {0, 1}.  Token t
  //      sees rows u in [max(t, W - 1 - pos0), min(t + W - 1, U - 1)] (positions
  //      max(0, pos0 + t - W + 1) .. pos0 + t).
  {
    const int pair = tid >> 4, j = tid & 15, t = pair >> 3;
    const int64_t lo64 = (int64_t)(W - 1) - pos0;
    const int lo = (int)(lo64 > t ? lo64 : t);
    const int hi = (t + W - 1 < U - 1) ? t + W - 1 : U - 1;
    const uint32_t span = (uint32_t)(hi - lo);                     // u visible <=> u - lo <= span (unsigned)
    constexpr int NC = kRows / 32;
    float z[2 * NC];
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int u = 2 * j + 32 * c;
      const float2 v2 = *reinterpret_cast<const float2*>(&l.s[pair][u]);
      z[2 * c] = (uint32_t)(u - lo) <= span ? v2.x : -__builtin_inff();
      z[2 * c + 1] = (uint32_t)(u + 1 - lo) <= span ? v2.y : -__builtin_inff();
      m = fmaxf(m, fmaxf(z[2 * c], z[2 * c + 1]));
    }
    m = row16_max(m);
    const float ms = m != -__builtin_inff() ? m : 0.0f;    // an empty row: every p = 0
    float lsum = 0.0f;
    uint32_t* ph = reinterpret_cast<uint32_t*>(&l.s[pair][0]);     // hi parts: bf16 [0, 168), lo: [168, 336)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float p0 = __builtin_amdgcn_exp2f(z[2 * c] - ms);       // exp2(-inf) = 0
      const float p1 = __builtin_amdgcn_exp2f(z[2 * c + 1] - ms);
      lsum += p0 + p1;
      const uint32_t h2 = pack_bf16x2(p0, p1);
      const uint32_t l2 = pack_bf16x2(p0 - __uint_as_float(h2 << 16), p1 - __uint_as_float(h2 & 0xffff0000u));
      ph[j + 16 * c] = h2;
      ph[kSStride / 2 + j + 16 * c] = l2;
    }
    lsum = row16_sum(lsum);
    if (j == 0) {
      const float sink2 = has_sink ? sinkv * 1.4426950408889634f : -__builtin_inff();
      const float M = fmaxf(m, sink2);
      float sc = 0.0f, den = 0.0f;
      if (M != -__builtin_inff()) {
        if (m != -__builtin_inff()) {
          sc = exp2f(m - M);
          den = lsum * sc;
        }
        if (sink2 != -__builtin_inff()) den += exp2f(sink2 - M);
      }
      l.scale[pair] = den > 0.0f ? sc / den : 0.0f;
    }
  }
  __syncthreads();
  DSA_MARK(trace, 4);
  // ---- 4) O = P V: wave w < 8 takes pairs 32 (w >> 2) .. +31 and dims 32 (w & 3) .. +31 as
  //      2 tiles of 32 x 32 (tile rows: 16 pairs x {hi, lo} parts; row m -> pair (m & 15),
  //      part m >> 4), K = 160 rows in 10 steps.  Two waves per SIMD hide each other's
  //      operand loads.
  if (wave < 8) {
    const int pb = wave >> 2, db = wave & 3;
    const int m = lane & 31;
    const int poff = ((m >> 4) * kSStride + 8 * (lane >> 5)) * 2;
    const uint8_t* pa0 = reinterpret_cast<const uint8_t*>(&l.s[pb * 32 + (m & 15)][0]) + poff;
    const uint8_t* pa1 = reinterpret_cast<const uint8_t*>(&l.s[pb * 32 + 16 + (m & 15)][0]) + poff;
    // transpose-load addresses: 16-lane group g covers dims +16 (g & 1) .. +15 of the tile and
    // rows 8 (g >> 1) .. +7 of the step; lane q of the group points at row (q >> 2), dims
    // 4 (q & 3) .. +3 (then 4 rows further for the second half)
    const int g = lane >> 4, q = lane & 15;
    const uint8_t* vb = l.v + (8 * (g >> 1) + (q >> 2)) * kRowB + (32 * db + 16 * (g & 1) + 4 * (q & 3)) * 2;
    f32x16_t acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < kRows / 16; ++ks) {
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
    uint16_t* xs = reinterpret_cast<uint16_t*>(l.k);
    const int dim = 32 * db + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int pbase = pb * 32 + mt * 16 + 4 * (lane >> 5);
      const float4 s0 = *reinterpret_cast<const float4*>(&l.scale[pbase]);
      const float4 s1 = *reinterpret_cast<const float4*>(&l.scale[pbase + 8]);
      const float scl[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pair = pbase + 8 * (e >> 2) + (e & 3);
        xs[(pair >> 3) * kXsStride + (pair & 7) * kD + dim] = f32_to_bf16((acc[mt][e] + acc[mt][e + 8]) * scl[e]);
      }
    }
  }
  __syncthreads();
  DSA_MARK(trace, 5);
}

// The W_o rows of output block b this lane multiplies (lane & 15 = row, lane >> 4 = k
// chunk of the wave's 64-wide k range).
template <bool F8>
struct WoFrags {
  static constexpr int NU = F8 ? 1 : 2;       // 16-byte units per lane
  Frag8 f[NU];
};

template <bool F8>
DSA_DEV void load_wo(int tid, const void* w_o, int b, WoFrags<F8>& wf) {
  constexpr int ESZ = F8 ? 1 : 2;
  constexpr int Kw = kOK / kWaves;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint4* wp = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(w_o) +
                                                   ((size_t)(b * kOutRows + (lane & 15)) * kOK + wave * Kw) * ESZ) +
                    (lane >> 4);
#pragma unroll
  for (int i = 0; i < WoFrags<F8>::NU; ++i) wf.f[i].u = wp[4 * i];
}

// Step 5: l.tile[r][t] = sum over k of W_o[16 b + r][k] * O[t][k] (the attention output in
// LDS), sixteen wave partials added in wave order; W8A8: per-token e4m3 quantisation of
// O first, and both scales applied to the sum (wsv: the scale of W_o row (tid >> 4) & 15).
template <bool F8>
DSA_DEV void oproj(int tid, const Lds& l, const WoFrags<F8>& wf, float wsv) {
  constexpr int Kw = kOK / kWaves;
  constexpr int XQS = kOK + 16;                // W8A8: LDS code row stride (bytes)
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw0 = wave * Kw;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(l.k);
  uint8_t* xq = l.v;     // W8A8 codes [kMaxT][XQS] (V is no longer needed)
  if constexpr (F8) {
    // per-token quantisation of the attention output: thread tid holds elements
    // 8 (tid & 127) .. +7 of token tid >> 7 (two waves per token)
    static_assert(kMaxT * kOK / 8 == kThreads && kMaxT * XQS <= kRows * kRowB, "one chunk per thread");
    const int t = tid >> 7, kk = (tid & 127) * 8;
    const uint4 y = *reinterpret_cast<const uint4*>(&xs[t * kXsStride + kk]);
    const uint32_t y4[4] = {y.x, y.y, y.z, y.w};
    const float m = row16_max(amax_bf16x8(y4));
    if ((lane & 15) == 0) l.amax[t][(wave & 1) * 4 + (lane >> 4)] = m;
    __syncthreads();
    if (wave < kMaxT) {             // wave t folds token t's eight partial maxima
      const float am = wave_max(lane < 8 ? l.amax[wave][lane] : 0.0f);
      if (lane == 0) {
        l.ainv[wave] = am > 0.0f ? 448.0f / am : 1.0f;
        l.ascale[wave] = am > 0.0f ? am / 448.0f : 1.0f;
      }
    }
    __syncthreads();
    *reinterpret_cast<uint2*>(xq + t * XQS + kk) = e4m3x8_scaled(y4, l.ainv[t]);
    __syncthreads();
  }
  float (*red)[16][16] = reinterpret_cast<float (*)[16][16]>(l.k + kMaxT * kXsStride * 2);
  {
    f32x4_t acc = {};
    const int tok = lane & 15;
#pragma unroll
    for (int j = 0; j < WoFrags<F8>::NU; ++j) {
      const int unit = 4 * j + (lane >> 4);
      Frag8 bfr;
      if (F8) bfr.u = *reinterpret_cast<const uint4*>(xq + (tok & 7) * XQS + kw0 + unit * 16);
      else bfr.u = *reinterpret_cast<const uint4*>(&xs[(tok & 7) * kXsStride + kw0 + unit * 8]);
      if (tok >= kMaxT) bfr.u = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (F8) {
        const Frag8 a = wf.f[j];
        const long a0 = (long)(((uint64_t)a.u.y << 32) | a.u.x), a1 = (long)(((uint64_t)a.u.w << 32) | a.u.z);
        const long b0 = (long)(((uint64_t)bfr.u.y << 32) | bfr.u.x), b1 = (long)(((uint64_t)bfr.u.w << 32) | bfr.u.z);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf.f[j].v, bfr.v, acc, 0, 0, 0);
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
    for (int w = 1; w < kWaves; ++w) v += red[w][r][c];
    if (F8) v *= l.ascale[c & 7] * wsv;             // W8A8: dequantise (columns >= T unused)
    l.tile[r][c] = v;
  }
  __syncthreads();
}


// ----------------------------------------------------------------------------- token groups
// The same steps for one group of G tokens (G = 2 or 4; group tg holds tokens G tg ..
// G tg + G - 1, i.e. pairs 8 G tg .. 8 G tg + 8 G - 1), for a workgroup that produces output
// columns of those tokens alone.  Every value is computed by the same instruction sequence
// at the same MFMA tile position as in the whole-block functions above: the score tile of
// pairs 32 q .. 32 q + 31 that holds the group (the other pairs' query rows zero), the P.V
// tiles of 16 pairs, the output-projection tiles of 16 W_o rows x 16 token columns (the
// other tokens' columns zero), partial sums added in the same order -- so the results are
// equal bit for bit.
// LDS: l.q holds the score tile's 32 query rows (column c = pair 32 q + c), l.s and l.scale
// the group's 8 G rows (row = pair - 8 G tg).

template <int G>
DSA_DEV void attention_group(int tid, const Lds& l, int tg, int64_t pos0, int W, int T, float sm_log2,
                             bool has_sink, float sinkv, uint64_t* trace) {
  static_assert(G == 2 || G == 4, "two or four tokens per group");
  constexpr int NP = 8 * G;                        // (token, head) rows of the group
  (void)trace;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int U = W + T - 1;
  const int p0 = NP * tg;                          // first pair of the group
  const int c0 = p0 & 31;                          // its first column in the score tile
  // ---- 2) scores: wave w < 5 takes rows 32 w .. 32 w + 31 against the tile's 32 columns;
  //      the group's columns go to LDS
  if (wave < kRows / 32) {
    const uint8_t* ka = l.k + (wave * 32 + (lane & 31)) * kRowB + (lane >> 5) * 16;
    const uint8_t* qa = l.q + (lane & 31) * kRowB + (lane >> 5) * 16;
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      Frag8 a, b0;
      a.u = *reinterpret_cast<const uint4*>(ka + ks * 32);
      b0.u = *reinterpret_cast<const uint4*>(qa + ks * 32);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b0.v, acc, 0, 0, 0);
    }
    const int pl = (lane & 31) - c0;
    if (pl >= 0 && pl < NP) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int u = wave * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        l.s[pl][u] = acc[e] * sm_log2;
      }
    }
  }
  __syncthreads();
  DSA_MARK(trace, 3);
  // ---- 3) softmax of the group's rows (16 lanes per row)
  if (tid < 16 * NP) {
    const int pl = tid >> 4, j = tid & 15, t = (p0 + pl) >> 3;
    const int64_t lo64 = (int64_t)(W - 1) - pos0;
    const int lo = (int)(lo64 > t ? lo64 : t);
    const int hi = (t + W - 1 < U - 1) ? t + W - 1 : U - 1;
    const uint32_t span = (uint32_t)(hi - lo);
    constexpr int NC = kRows / 32;
    float z[2 * NC];
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int u = 2 * j + 32 * c;
      const float2 v2 = *reinterpret_cast<const float2*>(&l.s[pl][u]);
      z[2 * c] = (uint32_t)(u - lo) <= span ? v2.x : -__builtin_inff();
      z[2 * c + 1] = (uint32_t)(u + 1 - lo) <= span ? v2.y : -__builtin_inff();
      m = fmaxf(m, fmaxf(z[2 * c], z[2 * c + 1]));
    }
    m = row16_max(m);
    const float ms = m != -__builtin_inff() ? m : 0.0f;
    float lsum = 0.0f;
    uint32_t* ph = reinterpret_cast<uint32_t*>(&l.s[pl][0]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float q0 = __builtin_amdgcn_exp2f(z[2 * c] - ms);
      const float q1 = __builtin_amdgcn_exp2f(z[2 * c + 1] - ms);
      lsum += q0 + q1;
      const uint32_t h2 = pack_bf16x2(q0, q1);
      const uint32_t l2 = pack_bf16x2(q0 - __uint_as_float(h2 << 16), q1 - __uint_as_float(h2 & 0xffff0000u));
      ph[j + 16 * c] = h2;
      ph[kSStride / 2 + j + 16 * c] = l2;
    }
    lsum = row16_sum(lsum);
    if (j == 0) {
      const float sink2 = has_sink ? sinkv * 1.4426950408889634f : -__builtin_inff();
      const float M = fmaxf(m, sink2);
      float sc = 0.0f, den = 0.0f;
      if (M != -__builtin_inff()) {
        if (m != -__builtin_inff()) {
          sc = exp2f(m - M);
          den = lsum * sc;
        }
        if (sink2 != -__builtin_inff()) den += exp2f(sink2 - M);
      }
      l.scale[pl] = den > 0.0f ? sc / den : 0.0f;
    }
  }
  __syncthreads();
  DSA_MARK(trace, 4);
  // ---- 4) O = P V: wave w < 4 takes dims 32 w .. +31 for the group's G / 2 tiles of 16
  //      pairs x {hi, lo} parts, K = 160 rows in 10 steps (one wave per SIMD: spreading the
  //      tiles over eight waves reads V twice and measured slower)
  if (wave < 4) {
    constexpr int MT = G / 2;
    const int db = wave;
    const int m = lane & 31;
    const int poff = ((m >> 4) * kSStride + 8 * (lane >> 5)) * 2;
    const int g = lane >> 4, q = lane & 15;
    const uint8_t* vb = l.v + (8 * (g >> 1) + (q >> 2)) * kRowB + (32 * db + 16 * (g & 1) + 4 * (q & 3)) * 2;
    f32x16_t acc[MT] = {};
#pragma unroll
    for (int ks = 0; ks < kRows / 16; ++ks) {
      Frag8 a[MT], bv;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[mt].u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(&l.s[16 * mt + (m & 15)][0]) +
                                                  poff + ks * 32);
      const uint2 lo4 = lds_tr16(vb + (16 * ks) * kRowB);
      const uint2 hi4 = lds_tr16(vb + (16 * ks + 4) * kRowB);
      bv.u = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt].v, bv.v, acc[mt], 0, 0, 0);
    }
    uint16_t* xs = reinterpret_cast<uint16_t*>(l.k);
    const int dim = 32 * db + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int pb = 16 * mt + 4 * (lane >> 5);     // row within the group, element e < 4
      const float4 s0 = *reinterpret_cast<const float4*>(&l.scale[pb]);
      const float4 s1 = *reinterpret_cast<const float4*>(&l.scale[pb + 8]);
      const float scl[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pair = p0 + pb + 8 * (e >> 2) + (e & 3);
        xs[(pair >> 3) * kXsStride + (pair & 7) * kD + dim] = f32_to_bf16((acc[mt][e] + acc[mt][e + 8]) * scl[e]);
      }
    }
  }
  __syncthreads();
  DSA_MARK(trace, 5);
}

// Step 5 for the 128 / G output columns (128 / G) cb .. + 128 / G - 1 (W_o row blocks
// (8 / G) cb + mt) and the token group tg.  Returns, for thread tid < 128, the sum of
// column row (128 / G) cb + tid / G for token G tg + tid % G (sixteen wave partials in
// wave order; W8A8: dequantised with the token's activation scale and wsv, the scale of
// that W_o row).
template <int G, bool F8>
DSA_DEV float oproj_group(int tid, const Lds& l, int tg, const WoFrags<F8> (&wf)[8 / G], float wsv) {
  constexpr int NMT = 8 / G;                       // W_o row tiles of 16
  constexpr int Kw = kOK / kWaves;
  constexpr int XQS = kOK + 16;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw0 = wave * Kw;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(l.k);
  uint8_t* xq = l.v;
  if constexpr (F8) {
    // per-token quantisation of the group's attention output: threads 0 .. 128 G - 1,
    // token G tg + (tid >> 7), elements 8 (tid & 127) .. +7 (two waves per token)
    if (tid < 128 * G) {
      const int t = G * tg + (tid >> 7), kk = (tid & 127) * 8;
      const uint4 y = *reinterpret_cast<const uint4*>(&xs[t * kXsStride + kk]);
      const uint32_t y4[4] = {y.x, y.y, y.z, y.w};
      const float m = row16_max(amax_bf16x8(y4));
      if ((lane & 15) == 0) l.amax[t][(wave & 1) * 4 + (lane >> 4)] = m;
    }
    __syncthreads();
    if (wave < G) {
      const int t = G * tg + wave;
      const float am = wave_max(lane < 8 ? l.amax[t][lane] : 0.0f);
      if (lane == 0) {
        l.ainv[t] = am > 0.0f ? 448.0f / am : 1.0f;
        l.ascale[t] = am > 0.0f ? am / 448.0f : 1.0f;
      }
    }
    __syncthreads();
    if (tid < 128 * G) {
      const int t = G * tg + (tid >> 7), kk = (tid & 127) * 8;
      const uint4 y = *reinterpret_cast<const uint4*>(&xs[t * kXsStride + kk]);
      const uint32_t y4[4] = {y.x, y.y, y.z, y.w};
      *reinterpret_cast<uint2*>(xq + t * XQS + kk) = e4m3x8_scaled(y4, l.ainv[t]);
    }
    __syncthreads();
  }
  float (*red)[16 * NMT][G] = reinterpret_cast<float (*)[16 * NMT][G]>(l.k + kMaxT * kXsStride * 2);
  {
    const int tok = lane & 15;
    const bool mine = tok / G == tg && tok < kMaxT;  // columns of other tokens are zero
    f32x4_t acc[NMT] = {};
#pragma unroll
    for (int j = 0; j < WoFrags<F8>::NU; ++j) {
      const int unit = 4 * j + (lane >> 4);
      Frag8 bfr;
      if (F8) bfr.u = *reinterpret_cast<const uint4*>(xq + (tok & 7) * XQS + kw0 + unit * 16);
      else bfr.u = *reinterpret_cast<const uint4*>(&xs[(tok & 7) * kXsStride + kw0 + unit * 8]);
      if (!mine) bfr.u = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        if constexpr (F8) {
          const Frag8 a = wf[mt].f[j];
          const long a0 = (long)(((uint64_t)a.u.y << 32) | a.u.x), a1 = (long)(((uint64_t)a.u.w << 32) | a.u.z);
          const long b0 = (long)(((uint64_t)bfr.u.y << 32) | bfr.u.x), b1 = (long)(((uint64_t)bfr.u.w << 32) | bfr.u.z);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, acc[mt], 0, 0, 0);
        } else {
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[mt].f[j].v, bfr.v, acc[mt], 0, 0, 0);
        }
      }
    }
    if (mine) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][16 * mt + 4 * (lane >> 4) + i][tok % G] = acc[mt][i];
    }
  }
  __syncthreads();
  float v = 0.0f;
  if (tid < 128) {
    const int r = tid / G, c = tid % G;
    v = red[0][r][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[w][r][c];
    if (F8) v *= l.ascale[G * tg + c] * wsv;
  }
  return v;
}

}  // namespace swa
}  // namespace dsa
