// Layer-step projections for gfx950: input RMSNorm + fused QKV/indexer projection with
// RoPE and cache append, and the output projection with the residual add.
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
// The projection arithmetic is in proj_core.h; this file holds the launches.
#include <cmath>

#include "dsa_common.h"
#include "dsa_kernels.h"
#include "proj_core.h"

namespace dsa {

template <int MODE, int NSTEP, bool R8, bool F8>
__global__ void __launch_bounds__(kProjThreads) proj_kernel(ProjParams p) {
  __shared__ ProjShared sh;
  proj_body<MODE, NSTEP, R8, F8, false, false>(threadIdx.x, p, proj_layer_of(p), blockIdx.x, sh, ProjTags{}, MODE == 0 ? p.trace : nullptr);
}

// workspace layout of the projection stage
constexpr size_t kWsKiStage = ctl::kBytes;
constexpr size_t kWsProjEnd = kWsKiStage + (size_t)kMaxT * kDI * sizeof(float);

hipError_t launch_proj_qkv(int kind, const void* x, const void* gamma, const void* w,
                           const float* wscale, int T, float eps, float theta, int64_t pos0,
                           void* qkv, void* q_att, void* q_idx, float* w_idx, void* kcache,
                           void* vcache, int64_t ring_cap, void* kidx, float* kidx_scale, void* ws,
                           hipStream_t st) {
  ProjParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = w;
  p.wscale = wscale;
  p.T = T;
  p.rpw = kind == 0 ? 16 : 8;                // DSA: 149 workgroups, SWA: 160 (one per CU)
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  p.kictr = reinterpret_cast<uint32_t*>(w8) + ctl::kDone;
  p.kistage = reinterpret_cast<float*>(w8 + kWsKiStage);
  p.gamma = static_cast<const uint16_t*>(gamma);
  p.eps = eps;
  p.theta = theta;
  for (int i = 0; i < kD / 2; ++i) p.inv_freq[i] = std::pow((double)theta, -2.0 * (double)i / (double)kD);
  for (int i = 0; i < kDI / 2; ++i) p.inv_freq[kD / 2 + i] = std::pow((double)theta, -2.0 * (double)i / (double)kDI);
  p.pos0 = pos0;
  p.qkv = static_cast<uint16_t*>(qkv);
  p.nproj = kind == 0 ? kNProjDSA : kNProjSWA;
  p.q_att = static_cast<uint16_t*>(q_att);
  p.q_idx = static_cast<uint16_t*>(q_idx);
  p.w_idx = w_idx;
  p.kcache = static_cast<uint16_t*>(kcache);
  p.vcache = static_cast<uint16_t*>(vcache);
  p.ring_cap = ring_cap;
  p.kidx = static_cast<uint8_t*>(kidx);
  p.kidx_scale = kidx_scale;
  const dim3 grid(proj_blocks(kind, p.rpw)), block(kProjThreads);
  // per-lane fragments: K / 8 waves / 4 lane groups / 8 = 16
#ifdef DSA_TRACE
  p.trace = dsa_trace_buffer() ? dsa_trace_buffer() + 512 * 16 : nullptr;   // rows 512.. of the buffer
#endif
  constexpr int nstep = kHidden / kProjWaves / 32;
  if (wscale) {
    if (p.rpw == 8) hipLaunchKernelGGL((proj_kernel<0, nstep, true, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((proj_kernel<0, nstep, false, true>), grid, block, 0, st, p);
  } else {
    if (p.rpw == 8) hipLaunchKernelGGL((proj_kernel<0, nstep, true, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((proj_kernel<0, nstep, false, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_proj_out(const void* o, const void* w_o, const float* wscale, const void* x,
                           void* xout, int T, void* ws, hipStream_t st) {
  (void)ws;
  ProjParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = w_o;
  p.wscale = wscale;
  p.o = static_cast<const uint16_t*>(o);
  p.xout = static_cast<uint16_t*>(xout);
  p.T = T;
  p.rpw = 16;
  const dim3 grid(kHidden / 16), block(kProjThreads);
  // 1024 / 8 waves / 4 lane groups / 8 = 4
  constexpr int nstep = kHq * kD / kProjWaves / 32;
  if (wscale) hipLaunchKernelGGL((proj_kernel<1, nstep, false, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((proj_kernel<1, nstep, false, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

size_t proj_workspace_bytes() { return kWsProjEnd; }

}  // namespace dsa
