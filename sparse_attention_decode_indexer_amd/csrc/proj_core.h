// Device code of the layer-step projections for gfx950: input RMSNorm + fused
// QKV/indexer projection with RoPE and cache append, and the output projection with the
// residual add.  Shared by the projection launches and the persistent multi-layer SWA
// kernel, so both compute the same bits.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §A DSA layer: from 29 kernels to one: input RMSNorm, Q/K/V projections, RoPE,
//     KV-cache writes, ..., output projection.
//   §Optimizing inside the kernel: projection weights do not depend on the normalised
//     input, so every projection workgroup issues its input and weight loads at entry
//     and normalises the block (and builds its rotary factors) while the weights stream
//     in.  Only the lanes of real weight rows issue weight loads.
//   §GPU Memory Optimization: positional-encoding precision at 1M context -- rotary
//     angles are formed in fp64.
//
// M = T <= 8 tokens makes these weight-streaming products.  One workgroup owns RPW rows
// of W (RPW = 4, 8 or 16, chosen so the launch covers the chip) over the full K; its
// sixteen waves split K.  A v_mfma_f32_16x16x32_bf16 tile takes the rows on the M side
// (rows >= RPW are never read) and the tokens on the N side (padded to 16).  Each lane
// streams its k chunks of one weight row straight into registers; the normalised
// activations sit in LDS.  The sixteen partial tiles are summed in wave order.
#pragma once
#include <cmath>

#include "dsa_common.h"

namespace dsa {

constexpr int kProjThreads = 1024;   // 16 waves: 4 per SIMD hide the load latency
constexpr int kProjWaves = kProjThreads / 64;
constexpr int kRowThreads = kHidden / 8;  // threads holding one token's 4096 inputs (8 each)

// Row block b of the fused projection for `rpw` rows per block.  Rotated segments are
// cut into blocks of rpw/2 rotary pairs (i, i + d/2) so RoPE is local to the block.
struct BlockInfo {
  int row0;     // first row of the first half (rotary) or of the block (plain)
  int rot_d;    // rotary width (128 or 64) or 0 for plain
  int i0;       // first pair index within the head (rotary)
  int seg;      // 0 Q, 1 K, 2 V, 3 q_I, 4 k_I, 5 w_I
};

// Segment table of the DSA projection [Q 1024 | K 128 | V 128 | q_I 1024 | k_I 64 | w_I 16]
// (SWA uses the first three).
DSA_DEV BlockInfo block_info(int b, int rpw) {
  const int hp = rpw / 2;                      // rotary pairs per block
  const int nq = kHq * (kD / 2) / hp;          // Q blocks
  const int nk = (kD / 2) / hp;                // K blocks
  const int nv = kD / rpw;                     // V blocks
  const int nqi = kHI * (kDI / 2) / hp;        // q_I blocks
  const int nki = (kDI / 2) / hp;              // k_I blocks
  BlockInfo bi;
  if (b < nq) {
    const int per_head = (kD / 2) / hp;
    const int h = b / per_head;
    bi.i0 = (b % per_head) * hp; bi.rot_d = kD; bi.row0 = h * kD + bi.i0; bi.seg = 0;
  } else if ((b -= nq) < nk) {
    bi.i0 = b * hp; bi.rot_d = kD; bi.row0 = kHq * kD + bi.i0; bi.seg = 1;
  } else if ((b -= nk) < nv) {
    bi.i0 = 0; bi.rot_d = 0; bi.row0 = kHq * kD + kD + b * rpw; bi.seg = 2;
  } else if ((b -= nv) < nqi) {
    const int per_head = (kDI / 2) / hp;
    const int h = b / per_head;
    bi.i0 = (b % per_head) * hp; bi.rot_d = kDI; bi.row0 = kHq * kD + 2 * kD + h * kDI + bi.i0; bi.seg = 3;
  } else if ((b -= nqi) < nki) {
    bi.i0 = b * hp; bi.rot_d = kDI; bi.row0 = kHq * kD + 2 * kD + kHI * kDI + bi.i0; bi.seg = 4;
  } else {
    b -= nki;
    bi.i0 = 0; bi.rot_d = 0; bi.row0 = kHq * kD + 2 * kD + kHI * kDI + kDI + b * rpw; bi.seg = 5;
  }
  return bi;
}

// weight row of local row r (0 .. rpw-1) of a block
DSA_DEV int block_row(const BlockInfo& bi, int r, int rpw) {
  if (bi.rot_d == 0) return bi.row0 + r;
  const int hp = rpw / 2;
  return r < hp ? bi.row0 + r : bi.row0 + bi.rot_d / 2 + (r - hp);
}

inline int proj_blocks(int kind, int rpw) {
  const int hp = rpw / 2;
  int n = kHq * (kD / 2) / hp + (kD / 2) / hp + kD / rpw;
  if (kind == 0) n += kHI * (kDI / 2) / hp + (kDI / 2) / hp + (kHI + rpw - 1) / rpw;
  return n;
}

struct ProjParams {
  const uint16_t* x;        // [T][4096] bf16 (QKV: layer input; OUT: residual input)
  const void* w;            // [N][K] bf16, or e4m3 codes (W8A8)
  const float* wscale;      // [N] fp32 dequantisation scale of each weight row (W8A8)
  int T;
  int rpw;                  // weight rows per workgroup
  // QKV
  const uint16_t* gamma;
  float eps;
  float theta;
  int64_t pos0;
  uint16_t* qkv;            // [T][N] bf16 post-RoPE (optional export)
  int nproj;
  uint16_t* q_att;          // [T][8][128] bf16 rotated queries
  uint16_t* q_idx;          // [T][16][64] bf16 rotated indexer queries (DSA)
  float* w_idx;             // [T][16] fp32 indexer head weights (DSA)
  uint16_t* kcache;         // [cap][128] bf16 (DSA) or ring
  uint16_t* vcache;
  int64_t ring_cap;         // 0 for a linear cache
  uint8_t* kidx;            // [cap][64] e4m3 (DSA)
  float* kidx_scale;
  uint32_t* kictr;          // counter of finished k_I blocks
  float* kistage;           // [T][64] rotated k_I values
  // OUT
  const uint16_t* o;        // [T][1024] bf16 attention output
  uint16_t* xout;           // [T][4096]
  uint64_t* trace;          // profiling builds: [blocks][16] phase timestamps
  // rotary inverse frequencies theta^(-2i/d) in fp64, formed on the host: [0, 64) for
  // width-128 heads, [64, 96) for width-64 indexer heads
  double inv_freq[kD / 2 + kDI / 2];
};

// The pointers that differ from layer to layer (the rest of ProjParams is shared)
struct ProjLayer {
  const uint16_t* x;        // QKV: the layer input [T][4096] (unless it arrives as tagged words)
  const void* w;            // weights (QKV [N][4096] or OUT [4096][1024])
  const uint16_t* gamma;    // QKV: RMSNorm weights [4096]
  uint16_t* kcache;         // QKV: K and V cache or ring
  uint16_t* vcache;
};

__host__ __device__ inline ProjLayer proj_layer_of(const ProjParams& p) {
  return ProjLayer{p.x, p.w, p.gamma, p.kcache, p.vcache};
}

// Tagged hand-offs of the persistent multi-layer SWA kernel: the layer input arrives as
// words xw (XT) and the rounded, rotated Q/K/V values also leave as words qw (QT), each
// word (tag << 32 | two bf16)
struct ProjTags {
  const uint64_t* xw;
  uint64_t* qw;
  uint32_t tag;
  uint32_t* ctl;            // the workspace's control words (error word on a timeout)
  float2 rot;               // ROTIN: (cos, sin) of thread (t = tid >> 3, pair tid & 7) < 64
};

constexpr int kXsStride = kHidden + 8;      // padded LDS row: rows fall in different banks

struct ProjShared {
  // normalised activations (QKV) or attention output (OUT): bf16, or for W8A8 their e4m3
  // codes in rows of kXsStride bytes
  alignas(16) uint16_t xs[kMaxT][kXsStride];
  alignas(16) float amax[kMaxT][32];           // W8A8: partial maxima of each token (16-lane rows)
  float ascale[kMaxT];                         // W8A8: activation scale of each token
  float ainv[kMaxT];                           // W8A8: 448 / amax of each token (1 for amax = 0)
  float red[kProjWaves][16][16];
  float tile[16][16];
  float rc[kMaxT][8];
  float rs[kMaxT][8];
  float rnorm[kMaxT];                          // 1 / rms of each token
  uint32_t last;
};

// Weights stream in 16-byte units: eight bf16 (one 16x16x32 bf16 step) or sixteen e4m3
// codes (two 16x16x32 fp8 steps).  Unit j of lane group g covers unit 4 j + g of the
// wave's k range, and the activation operand is read from the same unit.
// R8: eight weight rows per workgroup.  The MFMA still has 16 rows, so lanes 8..15 of
// each 16-lane group load the odd units of rows 0..7 (every load lane distinct) and a
// row rotate by 8 hands those units to lanes 0..7; MFMA rows 8..15 are never read.
// F8 (W8A8): e4m3 weights with a per-row scale; the activations are quantised per token
// to e4m3 on chip (see e4m3x8_scaled) and the fp32 products are scaled by both scales.
// Returns false when (XT) a wait for the layer input gave up; the workgroup then publishes
// no tagged words.
template <int MODE, int NSTEP, bool R8, bool F8, bool XT, bool QT, bool ROTIN = false>
DSA_DEV bool proj_body(int tid, const ProjParams& p, const ProjLayer& lp, int b, ProjShared& sh, const ProjTags& tg,
                       uint64_t* trace) {
  static_assert(!(XT || QT) || (MODE == 0 && R8 && !F8), "tagged hand-offs: bf16 QKV projection, 8 rows per block");
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int K = MODE == 0 ? kHidden : kHq * kD;    // reduction length (compile time: no divisions)
  constexpr int Kw = K / kProjWaves;                     // per wave (= NSTEP * 32)
  static_assert(Kw == NSTEP * 32, "each wave covers its k range in NSTEP steps of 32");
  constexpr int ESZ = F8 ? 1 : 2;                        // bytes per weight
  constexpr int NU = NSTEP * ESZ / 2;                    // 16-byte units per lane group
  constexpr int XQS = K + 16;                            // W8A8: LDS code row stride (bytes)
  uint8_t* const xq = reinterpret_cast<uint8_t*>(&sh.xs[0][0]);
  const int kw0 = wave * Kw;
  const int T = p.T;
  constexpr int rpw = R8 ? 8 : 16;           // p.rpw (the launch's), known at compile time
  const int lrow = lane & 15;
  BlockInfo bi{};
  int wrow;
  if (MODE == 0) {
    bi = block_info(b, rpw);
    wrow = block_row(bi, R8 ? (lrow & 7) : (lrow < rpw ? lrow : 0), rpw);
    if (bi.seg == 5 && wrow >= p.nproj) wrow = p.nproj - 1;   // partial last w_I block
  } else {
    wrow = b * rpw + (lrow < rpw ? lrow : 0);
  }
  // 1) activation loads first (needed first, and small), then all weight loads: the
  //    weights do not depend on the norm and stream in while it is computed.  Lane group
  //    g takes k chunk 4i+g of the wave's range at step i, so each load instruction reads
  //    64 contiguous bytes of every row.
  (void)trace;
  DSA_MARK(trace, 0);
  // QKV: the layer input x (normalised below); OUT: the attention output
  const uint16_t* src = MODE == 0 ? lp.x : p.o;
  constexpr int NCH = kMaxT * (MODE == 0 ? kHidden : kHq * kD) / 8 / kProjThreads;   // uint4 chunks per thread
  const int chunks = kMaxT * K / 8;
  uint4 v[NCH];
  float amx[NCH];                              // W8A8, QKV: running max |y| of each chunk
  if constexpr (!XT) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kProjThreads;
      const int cc = c < chunks ? c : chunks - 1;
      const int t = cc / (K / 8), kk = (cc % (K / 8)) * 8;
      const int tc = t < T ? t : T - 1;
      v[u] = *reinterpret_cast<const uint4*>(src + (size_t)tc * K + kk);
    }
  }
  uint4 gv = make_uint4(0u, 0u, 0u, 0u);
  if (MODE == 0) gv = reinterpret_cast<const uint4*>(lp.gamma)[tid % kRowThreads];   // gamma[8 j .. 8 j + 8)
  // OUT: the residual element this thread adds at the end, requested ahead of the weights
  uint16_t xres = 0;
  if (MODE == 1) {
    const int r = tid >> 4, t = tid & 15;
    if (tid < 256 && r < rpw && t < T) xres = p.x[(size_t)t * kHidden + b * rpw + r];
  }
  // W8A8: the scale of weight row (tid >> 4) & 15 of the block (the row this thread
  // dequantises in the tile reduction), requested before the weights
  float wsv = 1.0f;
  if constexpr (F8) {
    const int lr = (tid >> 4) & 15;
    int r;
    if (MODE == 0) {
      r = block_row(bi, lr < rpw ? lr : 0, rpw);
      r = r < p.nproj ? r : p.nproj - 1;
    } else {
      r = b * rpw + (lr < rpw ? lr : 0);
    }
    wsv = p.wscale[r];
  }
  // Every wave's activation requests go out before any wave's weight requests (an
  // execution barrier only: nothing waits for data), so the CU's return path serves the
  // block the norm needs first.  (Activations from tagged words: the weights go first and
  // stream in while the words are awaited.)
  if constexpr (!XT) __builtin_amdgcn_s_barrier();
  // Every lane loads (unconditional loads keep the wait counts exact): lanes beyond the
  // real rows repeat row 0's addresses, which the memory pipeline merges, and the MFMA
  // rows they feed are never read.
  constexpr int NW = R8 ? NU / 2 : NU;
  static_assert(!R8 || NU % 2 == 0, "R8 pairs the units");
  Frag8 wf[NW];
  {
    const uint4* wp = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(lp.w) +
                                                     ((size_t)wrow * K + kw0) * ESZ) +
                      (lane >> 4) + (R8 ? 4 * (lrow >> 3) : 0);
#pragma unroll
    for (int i = 0; i < NW; ++i) wf[i].u = wp[(R8 ? 8 : 4) * i];
  }
  bool xok = true;                             // XT: every awaited word arrived
  if constexpr (XT) {
    // the layer input as tagged words of two bf16 (x[t][2 i], x[t][2 i + 1]) = word t * 2048 + i,
    // 8 consecutive words from each of 256 producing workgroups.  First one word of each
    // producer (its last of the last token), so that waiting costs one load per producer
    // and round; then every word, most of them already there.
    if (tid < kHidden / 16) {
      uint32_t w1[1];
      xok = poll_words<1>([&](int) { return tg.xw + (size_t)(T - 1) * (kHidden / 2) + tid * 8 + 7; }, tg.tag, w1,
                          tg.ctl);
    }
    __syncthreads();
    // four words per 16-byte chunk, the chunks of the plain loads above
    uint32_t xw[4 * NCH];
    xok &= poll_words<4 * NCH>([&](int i) {
      const int c = tid + (i >> 2) * kProjThreads;
      const int cc = c < chunks ? c : chunks - 1;
      const int t = cc / (K / 8), kk = (cc % (K / 8)) * 8;
      const int tc = t < T ? t : T - 1;
      return tg.xw + (size_t)tc * (kHidden / 2) + kk / 2 + (i & 3);
    }, tg.tag, xw, tg.ctl);
#pragma unroll
    for (int u = 0; u < NCH; ++u) v[u] = make_uint4(xw[4 * u], xw[4 * u + 1], xw[4 * u + 2], xw[4 * u + 3]);
  }

  DSA_MARK(trace, 1);
  // rotary cos/sin of this block's pairs at the block's positions (first: it needs no
  // loaded data, so it runs while the loads are in flight): angle
  // (pos0 + t) * theta^(-2i/d) formed in fp64, cos/sin rounded to fp32.  The eight
  // inverse frequencies of the block are wave-uniform kernel arguments: scalar loads,
  // so no wait on the vector memory counter (which would also wait for the weights).
  if (MODE == 0 && bi.rot_d && tid < 8 * kMaxT && ROTIN) {
    // ROTIN: this thread's factors were computed by an earlier call of the same block
    const int t = tid >> 3, r = tid & 7;
    if (t < T && r < rpw / 2) {
      sh.rc[t][r] = tg.rot.x;
      sh.rs[t][r] = tg.rot.y;
    }
  } else if (MODE == 0 && bi.rot_d && tid < 8 * kMaxT) {
    const int t = tid >> 3, r = tid & 7;
    const int fbase = (bi.rot_d == kD ? 0 : kD / 2) + bi.i0;
    constexpr int NF = kD / 2 + kDI / 2;
    double inv = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double f = p.inv_freq[fbase + j < NF ? fbase + j : NF - 1];
      inv = r == j ? f : inv;
    }
    if (t < T && r < rpw / 2) {
      const double ang = (double)(p.pos0 + t) * inv;
      // Reduce by the nearest multiple of 2 pi first so sincos sees |x| <= pi (angles
      // reach ~1e6 rad at 1M context): 2 pi is split into fl(2 pi) and 2 pi - fl(2 pi),
      // each product removed by one fused multiply-add; the residual error (< 3e-16 rad)
      // is far below the fp32 rounding of cos and sin.
      const double kq = rint(ang * 0x1.45f306dc9c883p-3);                     // 1 / (2 pi)
      const double red = fma(-kq, 0x1.1a62633145c07p-52, fma(-kq, 0x1.921fb54442d18p+2, ang));
      double sv, cv;
      sincos(red, &sv, &cv);
      sh.rc[t][r] = (float)cv;
      sh.rs[t][r] = (float)sv;
    }
  }
  DSA_MARK(trace, 5);
  if (MODE == 0) {
    // Input RMSNorm while the weights stream in: thread tid holds elements [8 j, 8 j + 8),
    // j = tid mod 512, of tokens 2u + tid / 512 (u = 0..3).  Per token: squares summed in
    // element pairs per thread; thread partials go through LDS (the activation area, not
    // yet in use) and wave t adds token t's: lane i takes threads 8i .. 8i+7 in order,
    // then an xor butterfly over the wave.  y = bf16((x * gamma) * (1 / sqrt(mean + eps))).
    static_assert(MODE != 0 || (kProjWaves >= kMaxT && NCH * kProjThreads == kMaxT * kRowThreads), "norm layout");
    float* scr = reinterpret_cast<float*>(&sh.xs[0][0]);          // [kMaxT][kRowThreads]
    const int j8 = tid % kRowThreads;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int t = (tid + u * kProjThreads) / kRowThreads;
      const uint32_t x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float a2 = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, x4[q]);
        a2 = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, a2, false);     // exact squares, fp32 sum
      }
      scr[t * kRowThreads + j8] = a2;
    }
    // XT: a wait that gave up in any thread stops the workgroup's tagged outputs
    if constexpr (XT) xok = !__syncthreads_or(!xok);
    else __syncthreads();
    DSA_MARK(trace, 6);
    if (wave < kMaxT) {
      const float4 q0 = *reinterpret_cast<const float4*>(&scr[wave * kRowThreads + lane * 8]);
      const float4 q1 = *reinterpret_cast<const float4*>(&scr[wave * kRowThreads + lane * 8 + 4]);
      float a = ((((((q0.x + q0.y) + q0.z) + q0.w) + q1.x) + q1.y) + q1.z) + q1.w;
      // wave total in lane 0: DPP sums within rows of 16, then the row-pair and
      // half-wave swaps (a fixed order)
      a = row16_sum(a);
      {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        a = __uint_as_float(h[0]) + __uint_as_float(h[1]);
      }
      if (lane == 0) sh.rnorm[wave] = 1.0f / sqrtf(a / (float)kHidden + p.eps);
    }
    __syncthreads();
    DSA_MARK(trace, 7);
    // Rows of tokens >= T hold a copy of token T-1 (clamped loads): their products land
    // in MFMA columns that are never read.
    // x * gamma is exact in fp32 (a product of two bf16): one dot of the x pair with the
    // gamma pair whose other half is zero forms it, then one multiply by 1/rms
    const uint32_t g4[4] = {gv.x, gv.y, gv.z, gv.w};
    bf16x2_t glo[4], ghi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      glo[q] = __builtin_bit_cast(bf16x2_t, g4[q] & 0x0000ffffu);
      ghi[q] = __builtin_bit_cast(bf16x2_t, g4[q] & 0xffff0000u);
    }
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int t = (tid + u * kProjThreads) / kRowThreads;
      const float r = sh.rnorm[t];
      const uint32_t x4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t o4[4];
      amx[u] = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, x4[q]);
        const float y0 = __builtin_amdgcn_fdot2_f32_bf16(xv, glo[q], 0.0f, false) * r;
        const float y1 = __builtin_amdgcn_fdot2_f32_bf16(xv, ghi[q], 0.0f, false) * r;
        o4[q] = pack_bf16x2(y0, y1);
        if (F8) amx[u] = fmaxf(amx[u], fmaxf(fabsf(y0), fabsf(y1)));
      }
      v[u] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
      if (!F8) *reinterpret_cast<uint4*>(&sh.xs[t][8 * j8]) = v[u];
    }
  }
  // W8A8: partial maxima of |activation| per token, one per 16-lane row (chunk u of this
  // thread belongs to token (wave + 16 u) / WPT; WPT waves per token)
  constexpr int WPT = K / 8 / 64;                         // 8 (QKV) or 2 (OUT)
  if constexpr (F8) {
    static_assert(NCH * kProjThreads == kMaxT * K / 8 && WPT <= 8, "one chunk per (token, 8 elements)");
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const uint32_t y4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      // QKV: the chunk's fp32 max |y| rounded once equals the max of its rounded values
      // (round to nearest even is monotone and symmetric)
      const float m = row16_max(MODE == 0 ? round_bf16(amx[u]) : amax_bf16x8(y4));
      if ((lane & 15) == 0) sh.amax[(wave + 16 * u) / WPT][(wave % WPT) * 4 + (lane >> 4)] = m;
    }
  }
  // 2) activations into LDS (QKV bf16: already stored, normalised)
  if (MODE == 1 && !F8) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kProjThreads;
      if (c < chunks) {
        const int t = c / (K / 8), kk = (c % (K / 8)) * 8;
        *reinterpret_cast<uint4*>(&sh.xs[t][kk]) = t < T ? v[u] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __syncthreads();
  if constexpr (F8) {
    // W8A8: per-token quantisation of the activations held in v (the normalised input or
    // the attention output; rows of tokens >= T hold copies of token T-1 and feed MFMA
    // columns that are never read).  Wave t < 8 folds token t's 4 WPT partial maxima into
    // its scale and reciprocal; then every thread writes the eight codes of each chunk.
    if (wave < kMaxT) {
      const float am = wave_max(lane < 4 * WPT ? sh.amax[wave][lane] : 0.0f);
      if (lane == 0) {
        sh.ainv[wave] = am > 0.0f ? 448.0f / am : 1.0f;
        sh.ascale[wave] = am > 0.0f ? am / 448.0f : 1.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int t = (wave + 16 * u) / WPT;
      const uint32_t y4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const int kk = ((tid + u * kProjThreads) % (K / 8)) * 8;
      *reinterpret_cast<uint2*>(xq + t * XQS + kk) = e4m3x8_scaled(y4, sh.ainv[t]);
    }
    __syncthreads();
  }
  DSA_MARK(trace, 2);
  // 3) MFMA over this wave's k range
  f32x4_t acc = {};
  {
    const int tok = lane & 15;
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int unit = 4 * j + (lane >> 4);
      Frag8 bfr;
      if (F8) bfr.u = *reinterpret_cast<const uint4*>(xq + (tok & 7) * XQS + kw0 + unit * 16);
      else bfr.u = *reinterpret_cast<const uint4*>(&sh.xs[tok & 7][kw0 + unit * 8]);
      if (tok >= kMaxT) bfr.u = make_uint4(0u, 0u, 0u, 0u);
      Frag8 a;
      if constexpr (R8) {
        a = wf[j >> 1];
        if (j & 1) {          // odd unit: take lane (l + 8) mod 16 of the 16-lane row
          a.u.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.u.x, 0x128, 0xf, 0xf, true);
          a.u.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.u.y, 0x128, 0xf, 0xf, true);
          a.u.z = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.u.z, 0x128, 0xf, 0xf, true);
          a.u.w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.u.w, 0x128, 0xf, 0xf, true);
        }
      } else {
        a = wf[j];
      }
      if constexpr (F8) {
        // two k steps of 32 codes: bytes 0..7 and 8..15 of the unit
        const long a0 = (long)(((uint64_t)a.u.y << 32) | a.u.x), a1 = (long)(((uint64_t)a.u.w << 32) | a.u.z);
        const long b0 = (long)(((uint64_t)bfr.u.y << 32) | bfr.u.x), b1 = (long)(((uint64_t)bfr.u.w << 32) | bfr.u.z);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, bfr.v, acc, 0, 0, 0);
      }
    }
  }
  // D[row][tok]: lane holds tok = lane & 15, rows 4*(lane>>4) + i
#pragma unroll
  for (int i = 0; i < 4; ++i) sh.red[wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
  __syncthreads();
  if (tid < 256) {
    const int r = tid >> 4, c = tid & 15;
    float v = sh.red[0][r][c];
#pragma unroll
    for (int w = 1; w < kProjWaves; ++w) v += sh.red[w][r][c];
    if (F8) v *= sh.ascale[c & 7] * wsv;              // W8A8: dequantise (columns >= T unused)
    sh.tile[r][c] = v;
  }
  __syncthreads();
  DSA_MARK(trace, 3);
  // 4) epilogue
  if (MODE == 1) {
    // x_out[t][n] = bf16(x[t][n] + acc)
    const int r = tid >> 4, t = tid & 15;
    if (tid < 256 && r < rpw && t < T) {
      const size_t o = (size_t)t * kHidden + b * rpw + r;
      p.xout[o] = f32_to_bf16(sh.tile[r][t] + bf16_to_f32(xres));
    }
    return true;
  }
  // QKV: round, rotate pairs (r, r + rpw/2) at position pos0 + t, round, store
  DSA_MARK(trace, 4);
  const int hp = rpw / 2;
  if (tid < hp * kMaxT) {
    const int t = tid / hp, r = tid % hp;
    if (t < T) {
      const int64_t pos = p.pos0 + t;
      float a = round_bf16(sh.tile[r][t]);
      float c2 = round_bf16(sh.tile[r + hp][t]);
      if (bi.rot_d) {
        const float c = sh.rc[t][r], s = sh.rs[t][r];
        const float a2 = fmaf(-c2, s, a * c);
        const float b2 = fmaf(a, s, c2 * c);
        a = a2;
        c2 = b2;
      }
      const uint16_t ab = f32_to_bf16(a), bb = f32_to_bf16(c2);
      const int ra = block_row(bi, r, rpw), rb = block_row(bi, r + hp, rpw);
      const bool has_a = ra < p.nproj, has_b = rb < p.nproj;   // the last w_I block may be partial
      if (p.qkv) {
        uint16_t* q = p.qkv + (size_t)t * p.nproj;
        if (has_a) q[ra] = ab;
        if (has_b) q[rb] = bb;
      }
      // tagged hand-off: word t * 640 + 4 b + r carries rows (ra, rb) of token t
      if constexpr (QT)
        if (xok) ast64(tg.qw + (size_t)t * (kNProjSWA / 2) + b * 4 + r, ((uint64_t)tg.tag << 32) | ((uint32_t)bb << 16) | ab);
      if (bi.seg == 0 && !QT) {
        p.q_att[(size_t)t * kHq * kD + ra] = ab;
        p.q_att[(size_t)t * kHq * kD + rb] = bb;
      } else if (bi.seg == 3) {
        const int qb = kHq * kD + 2 * kD;
        p.q_idx[(size_t)t * kHI * kDI + ra - qb] = ab;
        p.q_idx[(size_t)t * kHI * kDI + rb - qb] = bb;
      } else if (bi.seg == 5) {
        const int wb = kHq * kD + 2 * kD + kHI * kDI + kDI;
        if (has_a) p.w_idx[t * kHI + ra - wb] = bf16_to_f32(ab);
        if (has_b) p.w_idx[t * kHI + rb - wb] = bf16_to_f32(bb);
      } else if (bi.seg == 1 || bi.seg == 2) {
        const int64_t slot = p.ring_cap ? pos % p.ring_cap : pos;
        uint16_t* dst = (bi.seg == 1 ? lp.kcache : lp.vcache) + slot * kD;
        const int base = (bi.seg == 1 ? kHq * kD : kHq * kD + kD);
        dst[ra - base] = ab;
        dst[rb - base] = bb;
      } else if (bi.seg == 4) {   // rotated k_I for the quantiser below (coherent stores)
        const int kib = kHq * kD + 2 * kD + kHI * kDI;
        astf(p.kistage + t * kDI + (ra - kib), bf16_to_f32(ab));
        astf(p.kistage + t * kDI + (rb - kib), bf16_to_f32(bb));
      }
    }
  }
  DSA_MARK(trace, 8);
  if (bi.seg != 4) return xok;
  // k_I: the last k_I block quantises the new rows (e4m3, per-row scale amax/448)
  vm_wait_all();
  __syncthreads();
  const uint32_t nki = (kDI / 2) / hp;
  if (tid == 0) sh.last = (aadd(p.kictr, 1u) == nki - 1u) ? 1u : 0u;
  __syncthreads();
  if (!sh.last) return true;
  if (wave < T) {                 // wave t: lane = dim
    const int t = wave, d = lane;
    const float v = aldf(p.kistage + t * kDI + d);
    const float am = wave_max(fabsf(v));
    const float scale = am > 0.0f ? am / 448.0f : 1.0f;
    const uint32_t code = f32_to_e4m3(v / scale);
    const int64_t pos = p.pos0 + t;
    p.kidx[pos * kDI + d] = (uint8_t)code;
    if (d == 0) p.kidx_scale[pos] = scale;
  }
  if (tid == 0) ast(p.kictr, 0u);
  return true;
}

}  // namespace dsa
