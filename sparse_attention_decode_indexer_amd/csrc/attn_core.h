// Device code of the split-K GQA attention shared by the attention kernels and the fused
// DSA layer kernel (one (token, split) per call, and the fixed-order split merge).
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §Model Architecture: attention runs only over the positions the indexer selected.
//   §Hybrid SWA-DSA Architecture: GQA (eight query heads of this GPU share one KV head),
//     a sink bias in both attention types.
//   §Optimizing inside the kernel: the selected K/V rows are staged on chip split by split
//     before the math; heads are the N side of a 16x16x32 MFMA, rows the M side.
#pragma once
#include "dsa_common.h"

namespace dsa {

constexpr int kAttnThreads = 256;
constexpr int kSplitRows = 64;
constexpr int kPartStride = 132;  // floats per (token, split, head): m, l, pad x2, acc[128]

struct AttnParams {
  const uint16_t* q;      // [T][8][128] bf16
  const uint8_t* kc;      // cache rows (bf16: 256 B, e4m3: 128 B)
  const uint8_t* vc;
  const float* ks;        // [rows] fp32 (e4m3 only)
  const float* vs;
  const int32_t* idx;     // MODE 0: [T][k]
  int k;
  int T;
  int64_t L;              // MODE 0: valid row range [0, L)
  int64_t ring_cap;       // MODE 1
  int64_t pos0;           // MODE 1
  int window;             // MODE 1
  float sm_log2;          // sm_scale * log2(e)
  const float* sink;      // [8] natural-log logits or nullptr
  void* out;
  int out_f32;
  uint64_t* trace;        // profiling builds: [blocks][16] phase timestamps
  float* part;            // [T][nsplit][8][kPartStride]
  int nsplit;
  // persistent launches (COH): results handed between the launch's workgroups as 64-bit
  // words (launch tag << 32 | 32-bit value), polled by the reader until the tag matches
  uint64_t* tpart;        // [T][nsplit][8][kTagPart] split partials: m, l, acc[128]
  uint64_t* tout;         // [T][512] the attention output, two bf16 per word
  uint32_t* ctl;          // the workspace's control words (error word on a wait that gives up)
};

constexpr int kTagPart = 2 + kD;   // tagged words per (token, split, head): m, l, acc[128]

// Word of dim d within a tagged partial: dims are stored (d % 4)-major, so the four
// stores of a thread holding dims 4 j .. 4 j + 3 each cover 32 consecutive words.
DSA_DEV int tag_dim_word(int d) { return 2 + (d & 3) * (kD / 4) + (d >> 2); }

template <int KVDT, int ROWS>
struct AttnShared {
  static constexpr int RB = KVDT == 0 ? 256 : 128;   // bytes per cache row
  static constexpr int KSTRIDE = RB + 16;            // padded K row stride
  int64_t rows[ROWS];
  alignas(16) uint8_t kst[ROWS * KSTRIDE];
  alignas(16) uint8_t vst[ROWS * RB];
  float kscl[ROWS];
  float vscl[ROWS];
  float s[kHq][ROWS];
};

// out[t][h][d4 .. d4+3] = o / den (0 for an empty list), fp32 or bf16; COH (bf16 only):
// two tagged words of the fused launch's attention output
template <bool COH>
DSA_DEV void store_out(const AttnParams& p, int t, int h, int d4, float (&o)[4], float den, uint32_t tag) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = den > 0.0f ? o[i] / den : 0.0f;
  const size_t ob = ((size_t)t * kHq + h) * kD + d4;
  if (COH) {
    const uint32_t w0 = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    const uint64_t tg = (uint64_t)tag << 32;
    ast64(p.tout + ob / 2, tg | w0);
    ast64(p.tout + ob / 2 + 1, tg | w1);
  } else if (p.out_f32) {
    float* of = static_cast<float*>(p.out) + ob;
    *reinterpret_cast<float4*>(of) = make_float4(o[0], o[1], o[2], o[3]);
  } else {
    uint16_t* ob16 = static_cast<uint16_t*>(p.out) + ob;
    const uint32_t w0 = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    *reinterpret_cast<uint2*>(ob16) = make_uint2(w0, w1);
  }
}

// One (token, split) of the attention by a workgroup of NT threads: the first 256 are
// (head = tid / 32, 4 dims); with NT = 512 or 1024 the P.V product is split over 2 or 4
// row groups whose partial sums are added in group order.  COH: the result (partial or
// final output) is written as tagged words, for a launch whose other workgroups consume
// it; the arithmetic is the same either way.
template <int KVDT, int MODE, int ROWS, int NT, bool COH>
DSA_DEV void attn_split(const AttnParams& p, int t, int split, AttnShared<KVDT, ROWS>& sh, uint64_t* trace,
                        uint32_t tag = 0u) {
  static_assert(ROWS % 64 == 0 && ROWS <= NT && NT % kAttnThreads == 0, "64-row blocks, one list entry per thread");
  constexpr int NW = NT / 64;                 // waves
  constexpr int G = NT / kAttnThreads;        // P.V row groups
  using SH = AttnShared<KVDT, ROWS>;
  constexpr int RB = SH::RB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  (void)trace;
  DSA_MARK(trace, 0);
  // ---- row list of this split
  if (tid < ROWS) {
    const int e = split * ROWS + tid;
    int64_t r = -1;
    if (MODE == 0) {
      if (e < p.k) {
        const int32_t v = p.idx[(size_t)t * p.k + e];
        if (v >= 0 && (int64_t)v < p.L) r = v;
      }
    } else {
      const int64_t pos = p.pos0 + t - p.window + 1 + e;
      if (e < p.window && pos >= 0) r = pos % p.ring_cap;
    }
    sh.rows[tid] = r;
    if (KVDT == 1) {
      const float ksv = p.ks[r >= 0 ? r : 0], vsv = p.vs[r >= 0 ? r : 0];
      sh.kscl[tid] = r >= 0 ? ksv : 0.0f;
      sh.vscl[tid] = r >= 0 ? vsv : 0.0f;
    }
  }
  __syncthreads();
  DSA_MARK(trace, 1);
  // ---- stage K and V rows (16-byte chunks, one row per RB/16 consecutive threads)
  {
    // every load is issued before any is consumed; invalid rows read row 0 and are zeroed
    constexpr int CPR = RB / 16;
    constexpr int NCH = ROWS * CPR / NT;
    uint4 kv[NCH], vv[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * NT;
      const int row = c / CPR, col = c % CPR;
      const int64_t r = sh.rows[row];
      const int64_t rr = r >= 0 ? r : 0;
      kv[u] = *reinterpret_cast<const uint4*>(p.kc + rr * RB + col * 16);
      vv[u] = *reinterpret_cast<const uint4*>(p.vc + rr * RB + col * 16);
    }
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * NT;
      const int row = c / CPR, col = c % CPR;
      const bool ok = sh.rows[row] >= 0;
      *reinterpret_cast<uint4*>(&sh.kst[row * SH::KSTRIDE + col * 16]) = ok ? kv[u] : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&sh.vst[row * RB + col * 16]) = ok ? vv[u] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // ---- q^T operand (heads on the N side): lane l -> head l%16 (< 8 real), dims kb*32 + (l/16)*8
  Frag8 qb[4];
  {
    const int h = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (h < kHq)
        qb[kb].u = *reinterpret_cast<const uint4*>(p.q + ((size_t)t * kHq + h) * kD + kb * 32 + (lane >> 4) * 8);
      else
        qb[kb].u = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  DSA_MARK(trace, 2);
  // ---- S = K q^T: wave w owns the 16-row blocks w, w + NW, ...
#pragma unroll
  for (int ib = 0; ib < (ROWS / 16 + NW - 1) / NW; ++ib) {
    const int rb16 = wave + ib * NW;
    if (rb16 >= ROWS / 16) break;
    f32x4_t acc = {};
    const int row = rb16 * 16 + (lane & 15);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag8 a;
      const int d0 = kb * 32 + (lane >> 4) * 8;
      if constexpr (KVDT == 0) {
        a.u = *reinterpret_cast<const uint4*>(&sh.kst[row * SH::KSTRIDE + d0 * 2]);
      } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(&sh.kst[row * SH::KSTRIDE + d0]);
        bf16x2_t x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, false);
        bf16x2_t x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, true);
        bf16x2_t x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, false);
        bf16x2_t x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, true);
        a.v = bf16x8_t{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, qb[kb].v, acc, 0, 0, 0);
    }
    const int h = lane & 15;
    if (h < kHq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = rb16 * 16 + (lane >> 4) * 4 + i;
        float z = acc[i];
        if (KVDT == 1) z *= sh.kscl[rr];
        sh.s[h][rr] = (sh.rows[rr] >= 0) ? z * p.sm_log2 : -__builtin_inff();
      }
    }
  }
  __syncthreads();
  DSA_MARK(trace, 3);
  // ---- softmax of the split: thread (h = tid/32, j = tid%32) holds rows j, j+32, ...
  constexpr int RPT = ROWS / 32;
  const int h = (tid >> 5) & (kHq - 1);
  const int jj = tid & 31;
  const int grp = tid / kAttnThreads;         // P.V row group
  const bool lead = grp == 0;
  float m = -__builtin_inff(), l = 0.0f;
  if (lead) {
    float z[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) z[i] = sh.s[h][jj + 32 * i];
    m = z[0];
#pragma unroll
    for (int i = 1; i < RPT; ++i) m = fmaxf(m, z[i]);
    // head h lives in one half-wave (rows 0-1 or 2-3 of 16 lanes): DPP row maxima, then
    // one row-pair swap
    m = row16_max(m);
    {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    float pz[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) pz[i] = 0.0f;
    if (m != -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) pz[i] = exp2f(z[i] - m);
    }
    l = pz[0];
#pragma unroll
    for (int i = 1; i < RPT; ++i) l += pz[i];
    // half-wave sum: DPP row sums and a row-pair swap; the association differs by lane, so
    // the half's first lane's total is broadcast to the half
    l = row16_sum(l);
    {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
      l = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 0));
      const float l1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 32));
      l = (lane & 32) ? l1 : l0;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if (KVDT == 1) pz[i] *= sh.vscl[jj + 32 * i];
      sh.s[h][jj + 32 * i] = pz[i];
    }
  }
  __syncthreads();
  DSA_MARK(trace, 4);
  // ---- acc[h][d4..d4+3] = sum_j p[h][j] * V[j][d4..d4+3]
  const int d4 = jj * 4;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // rows in groups of 8: the group's LDS reads are issued together
  constexpr int PVU = 8;
  constexpr int RG = ROWS / G;                // rows per group
  for (int j0 = grp * RG; j0 < (grp + 1) * RG; j0 += PVU) {
    float pj[PVU];
    float v[PVU][4];
#pragma unroll
    for (int u = 0; u < PVU; ++u) {
      const int j = j0 + u;
      pj[u] = sh.s[h][j];
      if constexpr (KVDT == 0) {
        const uint2 raw = *reinterpret_cast<const uint2*>(&sh.vst[j * RB + d4 * 2]);
        v[u][0] = __uint_as_float(raw.x << 16);
        v[u][1] = __uint_as_float(raw.x & 0xffff0000u);
        v[u][2] = __uint_as_float(raw.y << 16);
        v[u][3] = __uint_as_float(raw.y & 0xffff0000u);
      } else {
        const uint32_t raw = *reinterpret_cast<const uint32_t*>(&sh.vst[j * RB + d4]);
        auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw, false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw, true);
        v[u][0] = lo[0]; v[u][1] = lo[1]; v[u][2] = hi[0]; v[u][3] = hi[1];
      }
    }
#pragma unroll
    for (int u = 0; u < PVU; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(pj[u], v[u][i], acc[i]);
    }
  }
  if constexpr (G > 1) {
    // group partials through LDS (the K staging area is free now), added in group order
    float* pv = reinterpret_cast<float*>(sh.kst);                     // [G][kHq][kD]
    *reinterpret_cast<float4*>(&pv[(grp * kHq + h) * kD + d4]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (lead) {
#pragma unroll
      for (int g = 1; g < G; ++g) {
        const float4 q4 = *reinterpret_cast<const float4*>(&pv[(g * kHq + h) * kD + d4]);
        acc[0] += q4.x; acc[1] += q4.y; acc[2] += q4.z; acc[3] += q4.w;
      }
    }
  }
  DSA_MARK(trace, 5);
  float sink2 = -__builtin_inff();
  if (p.sink) sink2 = p.sink[h] * 1.4426950408889634f;
  if (p.nsplit == 1) {
    // the whole list in one workgroup: normalise here (same operations as the merge)
    const float M = fmaxf(m, sink2);
    float den = 0.0f;
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (M != -__builtin_inff()) {
      if (m != -__builtin_inff()) {
        const float sc = exp2f(m - M);
        den = fmaf(l, sc, den);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = fmaf(acc[i], sc, o[i]);
      }
      if (sink2 != -__builtin_inff()) den += exp2f(sink2 - M);
    }
    if (lead) store_out<COH>(p, t, h, d4, o, den, tag);
    DSA_MARK(trace, 6);
    return;
  }
  // ---- the split's partial (merged by the split merge)
  if (lead) {
    if (COH) {
      uint64_t* pw = p.tpart + (((size_t)t * p.nsplit + split) * kHq + h) * kTagPart;
      const uint64_t tg = (uint64_t)tag << 32;
      if (jj == 0) {
        ast64(pw, tg | __float_as_uint(m));
        ast64(pw + 1, tg | __float_as_uint(l));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ast64(pw + tag_dim_word(d4 + i), tg | __float_as_uint(acc[i]));
    } else {
      float* part = p.part + (((size_t)t * p.nsplit + split) * kHq + h) * kPartStride;
      if (jj == 0) *reinterpret_cast<float2*>(part) = make_float2(m, l);
      *reinterpret_cast<float4*>(part + 4 + d4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
  DSA_MARK(trace, 6);
}

}  // namespace dsa
