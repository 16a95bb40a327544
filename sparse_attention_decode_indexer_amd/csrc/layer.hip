// Layer-step projections for gfx950: input RMSNorm + fused QKV/indexer projection with
// RoPE and cache append, and the output projection with the residual add.
//
// Method: NaiveAI, "Naive-N0.5-Flash: Building Frontier AI with AI".
//   §A DSA layer: from 29 kernels to one: input RMSNorm, Q/K/V projections, RoPE,
//     KV-cache writes, ..., output projection.
//   §Optimizing inside the kernel: projection weights do not depend on the normalised
//     input, so every workgroup issues its weight loads first and computes RMSNorm of
//     the whole input locally while they are in flight (no global synchronisation
//     between the norm and the projection).
//   §GPU Memory Optimization: positional-encoding precision at 1M context -- rotary
//     angles are formed in fp64.
//
// M = T <= 8 tokens makes these weight-streaming products: one v_mfma_f32_16x16x32_bf16
// tile takes 16 output features (rows of W, the M side) against the tokens (the N side,
// padded to 16).  Each lane streams its own contiguous k range of one weight row straight
// into registers; the normalised activations sit in LDS.  K is split over the four waves
// of a workgroup and, when there are too few feature groups to cover the chip, over
// several workgroups whose partial tiles are summed in a fixed order by the last one.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kProjThreads = 256;
constexpr int kProjWaves = 4;

// Feature group g (16 rows of W) of the fused projection.  Rotated segments take 8 rotary
// pairs (i, i + d/2) per group so RoPE is local to the group.
struct GroupInfo {
  int row0;     // first row of the first 8 (rotary) or all 16 (plain) rows
  int rot_d;    // rotary width (128 or 64) or 0 for plain
  int i0;       // first pair index within the head (rotary)
  int seg;      // 0 Q, 1 K, 2 V, 3 q_I, 4 k_I, 5 w_I
};

DSA_DEV GroupInfo group_info(int g) {
  GroupInfo gi;
  if (g < 64) {                       // Q: 8 heads x 8 groups
    const int h = g >> 3;
    gi.i0 = (g & 7) * 8; gi.rot_d = kD; gi.row0 = h * kD + gi.i0; gi.seg = 0;
  } else if (g < 72) {                // K
    gi.i0 = (g - 64) * 8; gi.rot_d = kD; gi.row0 = kHq * kD + gi.i0; gi.seg = 1;
  } else if (g < 80) {                // V
    gi.i0 = 0; gi.rot_d = 0; gi.row0 = kHq * kD + kD + (g - 72) * 16; gi.seg = 2;
  } else if (g < 144) {               // q_I: 16 heads x 4 groups
    const int h = (g - 80) >> 2;
    gi.i0 = ((g - 80) & 3) * 8; gi.rot_d = kDI; gi.row0 = kHq * kD + 2 * kD + h * kDI + gi.i0; gi.seg = 3;
  } else if (g < 148) {               // k_I
    gi.i0 = (g - 144) * 8; gi.rot_d = kDI; gi.row0 = kHq * kD + 2 * kD + kHI * kDI + gi.i0; gi.seg = 4;
  } else {                            // w_I
    gi.i0 = 0; gi.rot_d = 0; gi.row0 = kHq * kD + 2 * kD + kHI * kDI + kDI; gi.seg = 5;
  }
  return gi;
}

// weight row of local row r (0..15) of a group
DSA_DEV int group_row(const GroupInfo& gi, int r) {
  if (gi.rot_d == 0) return gi.row0 + r;
  return r < 8 ? gi.row0 + r : gi.row0 + gi.rot_d / 2 + (r - 8);
}

struct ProjParams {
  // common
  const uint16_t* x;        // [T][4096] bf16 (QKV: layer input; OUT: residual input)
  const uint16_t* w;        // [N][K] bf16
  int T;
  int K;                    // reduction length (4096 QKV, 1024 OUT)
  int ks;                   // K split across workgroups
  int ngroups;
  float* part;              // [ngroups][ks][16][16]
  uint32_t* gctr;           // [ngroups] arrival counters
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
  uint32_t* kictr;          // counter of finished k_I groups
  float* kistage;           // [T][64] rotated k_I values
  // OUT
  const uint16_t* o;        // [T][1024] bf16 attention output
  uint16_t* xout;           // [T][4096]
};

struct ProjShared {
  alignas(16) uint16_t xs[kMaxT][kHidden];   // normalised activations (k range of this workgroup)
  float red[kProjWaves][16][16];
  float tile[16][16];
  float rsq[kMaxT];
  uint32_t last;
};

// Loads the A operand stream of this lane: row `wrow` of W, the lane group's contiguous
// k sub-range, NSTEP fragments of 8 bf16.
template <int NSTEP>
DSA_DEV void load_w_stream(const uint16_t* __restrict__ w, int K, int wrow, int kbeg, Frag8 (&f)[NSTEP]) {
  const uint4* p = reinterpret_cast<const uint4*>(w + (size_t)wrow * K + kbeg);
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) f[i].u = p[i];
}

template <int MODE, int NSTEP>
__global__ void __launch_bounds__(kProjThreads) proj_kernel(ProjParams p) {
  __shared__ ProjShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = blockIdx.x / p.ks;
  const int kpart = blockIdx.x % p.ks;
  const int Kr = p.K / p.ks;                 // k range of this workgroup
  const int k0 = kpart * Kr;
  const int Kw = Kr / kProjWaves;            // per wave
  const int kw0 = k0 + wave * Kw;
  const int sub = Kw / 4;                    // per lane group (= NSTEP * 8)
  const int T = p.T;
  GroupInfo gi;
  int wrow;
  if (MODE == 0) {
    gi = group_info(g);
    wrow = group_row(gi, lane & 15);
  } else {
    wrow = g * 16 + (lane & 15);
  }
  // 1) weights first: they do not depend on the norm
  Frag8 wf[NSTEP];
  load_w_stream<NSTEP>(p.w, p.K, wrow, kw0 + (lane >> 4) * sub, wf);
  // 2) activations of this workgroup's k range into LDS
  if (MODE == 0) {
    // RMSNorm statistics over the full row: 32 threads per token, fixed order
    const int t = tid >> 5, j = tid & 31;
    float ss = 0.0f;
    if (t < T) {
      const uint4* xr = reinterpret_cast<const uint4*>(p.x + (size_t)t * kHidden);
      for (int c = j; c < kHidden / 8; c += 32) {
        const uint4 v = xr[c];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = __uint_as_float(w4[q] << 16), b = __uint_as_float(w4[q] & 0xffff0000u);
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        }
      }
    }
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, 64);
    if (j == 0 && t < kMaxT) sh.rsq[t] = (t < T) ? 1.0f / sqrtf(ss / (float)kHidden + p.eps) : 0.0f;
    __syncthreads();
    for (int c = tid; c < kMaxT * Kr / 2; c += kProjThreads) {
      const int t2 = c / (Kr / 2), kk = (c % (Kr / 2)) * 2;
      uint32_t outw = 0u;
      if (t2 < T) {
        const uint32_t xv = *reinterpret_cast<const uint32_t*>(p.x + (size_t)t2 * kHidden + k0 + kk);
        const uint32_t gv = *reinterpret_cast<const uint32_t*>(p.gamma + k0 + kk);
        const float r = sh.rsq[t2];
        const float y0 = (__uint_as_float(xv << 16) * r) * __uint_as_float(gv << 16);
        const float y1 = (__uint_as_float(xv & 0xffff0000u) * r) * __uint_as_float(gv & 0xffff0000u);
        outw = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
      }
      *reinterpret_cast<uint32_t*>(&sh.xs[t2][kk]) = outw;
    }
  } else {
    for (int c = tid; c < kMaxT * Kr / 8; c += kProjThreads) {
      const int t2 = c / (Kr / 8), kk = (c % (Kr / 8)) * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t2 < T) v = *reinterpret_cast<const uint4*>(p.o + (size_t)t2 * p.K + k0 + kk);
      *reinterpret_cast<uint4*>(&sh.xs[t2][kk]) = v;
    }
  }
  __syncthreads();
  // 3) MFMA over this wave's k range
  f32x4_t acc = {};
  {
    const int tok = lane & 15;
    const int kl = (kw0 - k0) + (lane >> 4) * sub;   // local k of this lane group
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      Frag8 b;
      if (tok < kMaxT) b.u = *reinterpret_cast<const uint4*>(&sh.xs[tok][kl + i * 8]);
      else b.u = make_uint4(0u, 0u, 0u, 0u);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i].v, b.v, acc, 0, 0, 0);
    }
  }
  // D[row][tok]: lane holds tok = lane & 15, rows 4*(lane>>4) + i
#pragma unroll
  for (int i = 0; i < 4; ++i) sh.red[wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
  __syncthreads();
  {
    const int r = tid >> 4, c = tid & 15;
    float v = sh.red[0][r][c];
#pragma unroll
    for (int w = 1; w < kProjWaves; ++w) v += sh.red[w][r][c];
    sh.tile[r][c] = v;
  }
  __syncthreads();
  // 4) split-K: the last workgroup of the group sums the partial tiles in order
  if (p.ks > 1) {
    float* mine = p.part + ((size_t)g * p.ks + kpart) * 256;
    astf(mine + tid, sh.tile[tid >> 4][tid & 15]);
    vm_wait_all();
    __syncthreads();
    if (tid == 0) sh.last = (aadd(p.gctr + g, 1u) == (uint32_t)p.ks - 1u) ? 1u : 0u;
    __syncthreads();
    if (!sh.last) return;
    float v = 0.0f;
    for (int s = 0; s < p.ks; ++s) v += aldf(p.part + ((size_t)g * p.ks + s) * 256 + tid);
    __syncthreads();
    sh.tile[tid >> 4][tid & 15] = v;
    if (tid == 0) ast(p.gctr + g, 0u);
    __syncthreads();
  }
  // 5) epilogue
  if (MODE == 1) {
    // x_out[t][n] = bf16(x[t][n] + acc)
    const int r = tid >> 4, t = tid & 15;
    if (t < T) {
      const size_t o = (size_t)t * kHidden + g * 16 + r;
      const float xr = bf16_to_f32(p.x[o]);
      p.xout[o] = f32_to_bf16(sh.tile[r][t] + xr);
    }
    return;
  }
  // QKV: round, rotate pairs (r, r+8) at position pos0 + t, round, store
  if (tid < 8 * kMaxT) {
    const int t = tid >> 3, r = tid & 7;
    if (t < T) {
      const int64_t pos = p.pos0 + t;
      float a = round_bf16(sh.tile[r][t]);
      float b = round_bf16(sh.tile[r + 8][t]);
      if (gi.rot_d) {
        const int i = gi.i0 + r;
        const double inv = pow((double)p.theta, -2.0 * (double)i / (double)gi.rot_d);
        const double ang = (double)pos * inv;
        const float c = (float)cos(ang), s = (float)sin(ang);
        const float a2 = fmaf(-b, s, a * c);
        const float b2 = fmaf(a, s, b * c);
        a = a2;
        b = b2;
      }
      const uint16_t ab = f32_to_bf16(a), bb = f32_to_bf16(b);
      const int ra = group_row(gi, r), rb = group_row(gi, r + 8);
      if (p.qkv) {
        uint16_t* q = p.qkv + (size_t)t * p.nproj;
        q[ra] = ab;
        q[rb] = bb;
      }
      if (gi.seg == 0) {
        p.q_att[(size_t)t * kHq * kD + ra] = ab;
        p.q_att[(size_t)t * kHq * kD + rb] = bb;
      } else if (gi.seg == 3) {
        const int qb = kHq * kD + 2 * kD;
        p.q_idx[(size_t)t * kHI * kDI + ra - qb] = ab;
        p.q_idx[(size_t)t * kHI * kDI + rb - qb] = bb;
      } else if (gi.seg == 5) {
        const int wb = kHq * kD + 2 * kD + kHI * kDI + kDI;
        p.w_idx[t * kHI + ra - wb] = bf16_to_f32(ab);
        p.w_idx[t * kHI + rb - wb] = bf16_to_f32(bb);
      }
      if (gi.seg == 1 || gi.seg == 2) {
        const int64_t slot = p.ring_cap ? pos % p.ring_cap : pos;
        uint16_t* dst = (gi.seg == 1 ? p.kcache : p.vcache) + slot * kD;
        const int base = (gi.seg == 1 ? kHq * kD : kHq * kD + kD);
        dst[ra - base] = ab;
        dst[rb - base] = bb;
      }
      if (gi.seg == 4) {      // rotated k_I values for the quantiser below (coherent stores)
        const int kib = kHq * kD + 2 * kD + kHI * kDI;
        astf(p.kistage + t * kDI + (ra - kib), bf16_to_f32(ab));
        astf(p.kistage + t * kDI + (rb - kib), bf16_to_f32(bb));
      }
    }
  }
  if (gi.seg != 4) return;
  // k_I: the last of the four k_I groups quantises the new rows (e4m3, scale amax/448)
  vm_wait_all();
  __syncthreads();
  if (tid == 0) sh.last = (aadd(p.kictr, 1u) == 3u) ? 1u : 0u;
  __syncthreads();
  if (!sh.last) return;
  if (tid < 64 * kMaxT) {
    // one wave per token: lane = dim
    for (int t = wave; t < T; t += kProjWaves) {
      const int d = lane;
      const float v = aldf(p.kistage + t * kDI + d);
      float am = fabsf(v);
#pragma unroll
      for (int dd = 32; dd >= 1; dd >>= 1) am = fmaxf(am, __shfl_xor(am, dd, 64));
      const float scale = am > 0.0f ? am / 448.0f : 1.0f;
      const uint32_t code = f32_to_e4m3(v / scale);
      const int64_t pos = p.pos0 + t;
      p.kidx[pos * kDI + d] = (uint8_t)code;
      if (d == 0) p.kidx_scale[pos] = scale;
    }
  }
  if (tid == 0) ast(p.kictr, 0u);
}

hipError_t launch_proj_qkv(int kind, const void* x, const void* gamma, const void* w, int T,
                           float eps, float theta, int64_t pos0, void* qkv, void* q_att,
                           void* q_idx, float* w_idx, void* kcache, void* vcache,
                           int64_t ring_cap, void* kidx, float* kidx_scale, void* ws,
                           hipStream_t st) {
  ProjParams p{};
  p.q_att = static_cast<uint16_t*>(q_att);
  p.q_idx = static_cast<uint16_t*>(q_idx);
  p.w_idx = w_idx;
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(w);
  p.T = T;
  p.K = kHidden;
  p.ngroups = kind == 0 ? 149 : 80;
  p.ks = kind == 0 ? 2 : 4;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  p.gctr = reinterpret_cast<uint32_t*>(w8) + ctl::kWords;   // inside the 8 KiB control block
  p.kictr = reinterpret_cast<uint32_t*>(w8) + ctl::kDone;
  p.part = reinterpret_cast<float*>(w8 + ctl::kBytes);
  p.kistage = reinterpret_cast<float*>(w8 + ctl::kBytes + (size_t)149 * 4 * 256 * sizeof(float));
  p.gamma = static_cast<const uint16_t*>(gamma);
  p.eps = eps;
  p.theta = theta;
  p.pos0 = pos0;
  p.qkv = static_cast<uint16_t*>(qkv);
  p.nproj = kind == 0 ? kNProjDSA : kNProjSWA;
  p.kcache = static_cast<uint16_t*>(kcache);
  p.vcache = static_cast<uint16_t*>(vcache);
  p.ring_cap = ring_cap;
  p.kidx = static_cast<uint8_t*>(kidx);
  p.kidx_scale = kidx_scale;
  const dim3 grid(p.ngroups * p.ks), block(kProjThreads);
  // per-lane fragments: K / ks / 4 waves / 4 lane groups / 8
  if (p.ks == 2) hipLaunchKernelGGL((proj_kernel<0, 16>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((proj_kernel<0, 8>), grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_proj_out(const void* o, const void* w_o, const void* x, void* xout, int T,
                           void* ws, hipStream_t st) {
  ProjParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(w_o);
  p.o = static_cast<const uint16_t*>(o);
  p.xout = static_cast<uint16_t*>(xout);
  p.T = T;
  p.K = kHq * kD;
  p.ks = 1;
  p.ngroups = kHidden / 16;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  p.gctr = reinterpret_cast<uint32_t*>(w8) + ctl::kWords;
  p.part = reinterpret_cast<float*>(w8 + ctl::kBytes);
  const dim3 grid(p.ngroups), block(kProjThreads);
  hipLaunchKernelGGL((proj_kernel<1, 8>), grid, block, 0, st, p);
  return hipGetLastError();
}

size_t proj_workspace_bytes() {
  return ctl::kBytes + (size_t)149 * 4 * 256 * sizeof(float) + (size_t)kMaxT * kDI * sizeof(float);
}

}  // namespace dsa
