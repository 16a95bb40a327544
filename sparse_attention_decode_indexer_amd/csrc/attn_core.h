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
  static constexpr int VRB = kD * 2 + 16;            // staged V rows: bf16 (e4m3 converted), padded
                                                     // so the transpose reads of 4 rows hit distinct banks
  static constexpr int PSTR = ROWS + 8;              // bf16 per row of a P part (padded)
  static constexpr int OXS = kD + 4;                 // floats per head of the P.V exchange
  int64_t rows[ROWS];
  // K rows; after the scores: P in three bf16 parts [3][kHq][PSTR], then the P.V result
  // [kHq][OXS] fp32
  alignas(16) uint8_t kst[ROWS * KSTRIDE];
  alignas(16) uint8_t vst[ROWS * VRB];
  float kscl[ROWS];
  float vscl[ROWS];
  float s[kHq][ROWS];
  static_assert(3 * kHq * PSTR * 2 % 16 == 0 && 3 * kHq * PSTR * 2 + kHq * OXS * 4 <= ROWS * KSTRIDE,
                "P parts and the P.V result fit the K staging area");
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

// One (token, split) of the attention by a workgroup of NT threads: every thread stages
// rows; the first 256 run the softmax and write the result as (head = tid / 32, 4 dims);
// four waves form P.V on the matrix cores.  COH: the result (partial or final output) is
// written as tagged words, for a launch whose other workgroups consume it; the arithmetic
// is the same either way.
template <int KVDT, int MODE, int ROWS, int NT, bool COH>
DSA_DEV void attn_split(const AttnParams& p, int t, int split, AttnShared<KVDT, ROWS>& sh, uint64_t* trace,
                        uint32_t tag = 0u) {
  static_assert(ROWS % 64 == 0 && ROWS <= NT && NT % kAttnThreads == 0, "64-row blocks, one list entry per thread");
  constexpr int NW = NT / 64;                 // waves
  static_assert(NW >= kD / 32, "four waves for the P.V tiles");
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
      // component-wise selects (a select of two uint4 objects went through scratch)
      auto keep = [ok](const uint4& v) {
        return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
      };
      *reinterpret_cast<uint4*>(&sh.kst[row * SH::KSTRIDE + col * 16]) = keep(kv[u]);
      if constexpr (KVDT == 0) {
        *reinterpret_cast<uint4*>(&sh.vst[row * SH::VRB + col * 16]) = keep(vv[u]);
      } else {
        // sixteen e4m3 codes -> sixteen bf16 (exact), the P.V operand's format
        const uint32_t cw[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        uint32_t bw[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cw[w], 1.0f, false);
          const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cw[w], 1.0f, true);
          bw[2 * w] = __builtin_bit_cast(uint32_t, a);
          bw[2 * w + 1] = __builtin_bit_cast(uint32_t, b);
        }
        *reinterpret_cast<uint4*>(&sh.vst[row * SH::VRB + col * 32]) = keep(make_uint4(bw[0], bw[1], bw[2], bw[3]));
        *reinterpret_cast<uint4*>(&sh.vst[row * SH::VRB + col * 32 + 16]) =
            keep(make_uint4(bw[4], bw[5], bw[6], bw[7]));
      }
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
  const bool lead = tid < kAttnThreads;       // the softmax and result threads
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
    // P in three bf16 parts, P = hi + mid + lo exactly (8 + 8 + 8 significant bits of
    // the fp32 value; each residual is exact in fp32), the A operand of the P.V product
    uint16_t* pp = reinterpret_cast<uint16_t*>(sh.kst);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if (KVDT == 1) pz[i] *= sh.vscl[jj + 32 * i];
      const uint16_t b0 = f32_to_bf16(pz[i]);
      const float r1 = pz[i] - bf16_to_f32(b0);
      const uint16_t b1 = f32_to_bf16(r1);
      const uint16_t b2 = f32_to_bf16(r1 - bf16_to_f32(b1));
      const int j = jj + 32 * i;
      pp[(0 * kHq + h) * SH::PSTR + j] = b0;
      pp[(1 * kHq + h) * SH::PSTR + j] = b1;
      pp[(2 * kHq + h) * SH::PSTR + j] = b2;
    }
  }
  __syncthreads();
  DSA_MARK(trace, 4);
  // ---- O = P V on the matrix cores: wave w < 4 takes dims 32 w .. +31 as one 32 x 32 tile
  //      whose rows are (part, head) = (m >> 3, m & 7) for m < 24 (rows 24-31 zero),
  //      K = the split's rows in steps of 16; V through the LDS transpose path.  The
  //      products are exact and accumulate in fp32; the three parts of each head are added
  //      (hi + mid) + lo and the result goes through LDS to the softmax's thread layout.
  float* ox = reinterpret_cast<float*>(sh.kst + 3 * kHq * SH::PSTR * 2);   // [kHq][OXS]
  if (wave < kD / 32) {
    const int m = lane & 31;
    const uint8_t* pa = sh.kst + (m * SH::PSTR + 8 * (lane >> 5)) * 2;
    const int g = lane >> 4, q = lane & 15;
    const uint8_t* vb = sh.vst + (8 * (g >> 1) + (q >> 2)) * SH::VRB + (32 * wave + 16 * (g & 1) + 4 * (q & 3)) * 2;
    f32x16_t pv = {};
#pragma unroll
    for (int ks = 0; ks < ROWS / 16; ++ks) {
      Frag8 a, bv;
      a.u = make_uint4(0u, 0u, 0u, 0u);
      if (m < 3 * kHq) a.u = *reinterpret_cast<const uint4*>(pa + ks * 32);
      const uint2 lo4 = lds_tr16(vb + (16 * ks) * SH::VRB);
      const uint2 hi4 = lds_tr16(vb + (16 * ks + 4) * SH::VRB);
      bv.u = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
      pv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, bv.v, pv, 0, 0, 0);
    }
    // lane l, element e < 4: head 4 (l >> 5) + e, part 0; elements e + 4, e + 8: parts 1, 2
    const int dim = 32 * wave + (lane & 31);
#pragma unroll
    for (int e = 0; e < 4; ++e) ox[(4 * (lane >> 5) + e) * SH::OXS + dim] = (pv[e] + pv[e + 4]) + pv[e + 8];
  }
  __syncthreads();
  const int d4 = jj * 4;
  float acc[4];
  {
    const float4 o4 = *reinterpret_cast<const float4*>(&ox[h * SH::OXS + d4]);
    acc[0] = o4.x; acc[1] = o4.y; acc[2] = o4.z; acc[3] = o4.w;
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
