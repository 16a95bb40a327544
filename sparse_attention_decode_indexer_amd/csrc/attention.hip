// Split-K GQA attention over a list of cache rows, for gfx950.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
//   §Model Architecture: attention runs only over the positions the indexer selected.
//   §Hybrid SWA-DSA Architecture: GQA (eight query heads of this GPU share one KV head),
//     a 128-token sliding window for SWA layers, a sink bias in both attention types.
//   §Optimizing inside the kernel: the selected K/V rows are staged on chip split by split
//     before the math; the eight heads are mapped so the matrix unit is not padded by
//     heads (here: heads are the N side of a 16x16x32 MFMA, rows the M side).
//
// One workgroup = one (token, split of 64 list entries).  It stages the split's K and V
// rows in LDS with 16-byte coalesced loads, computes S = K q^T on the matrix cores,
// runs the softmax of the split in fp32 (base-2 exponentials of log2e-scaled logits),
// forms P V on the matrix cores (P split exactly into three bf16 parts, fp32
// accumulation), and writes (m, l, acc) to the workspace.  A second, small kernel
// merges each token's splits in split order (the kernel boundary makes the partials
// visible), so the result does not depend on timing.
#include "attn_core.h"
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

template <int KVDT, int MODE, int ROWS, int NT>
__global__ void __launch_bounds__(NT) attn_kernel(AttnParams p) {
  __shared__ AttnShared<KVDT, ROWS> sh;
  const int split = blockIdx.x;
  const int t = blockIdx.y;
  uint64_t* trace = p.trace ? p.trace + (size_t)(t * gridDim.x) * 16 : nullptr;   // row = block index
  attn_split<KVDT, MODE, ROWS, NT, false>(p, t, split, sh, trace);
}

// Merge of token t's splits for one output slice (head slice >> 2, dims 32 (slice & 3)
// ..+31), one wave: lane j holds split j's (m, l); lane i < 32 holds dim i of every split.
// Splits are combined in split order; empty splits (m = -inf) are skipped.
__global__ void __launch_bounds__(64) attn_merge_kernel(AttnParams p) {
  const int lane = threadIdx.x;
  const int slice = blockIdx.x;
  const int t = blockIdx.y;
  const int ns = p.nsplit;
  const int hh = slice >> 2, d0 = (slice & 3) * 32;
  const int jl = lane & 31;
  const float* pt = p.part + (size_t)t * ns * kHq * kPartStride;
  const int jc = jl < ns ? jl : ns - 1;
  const float2 ml = *reinterpret_cast<const float2*>(pt + ((size_t)jc * kHq + hh) * kPartStride);
  float a[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int js = j < ns ? j : ns - 1;
    a[j] = pt[((size_t)js * kHq + hh) * kPartStride + 4 + d0 + jl];
  }
  const float mj = jl < ns ? ml.x : -__builtin_inff();
  const float mr = row16_max(mj);                          // rows of 16 lanes, then the two rows
  float M = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 0)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 16)));
  float s2 = -__builtin_inff();
  if (p.sink) s2 = p.sink[hh] * 1.4426950408889634f;
  M = fmaxf(M, s2);
  // split j's rescale factor (0 for empty or missing splits, whose accumulators are 0) and
  // denominator go through LDS, so every lane walks the splits in order without lane moves
  __shared__ float wsc[32], lsc[32];
  if (lane < 32) {
    wsc[lane] = (M != -__builtin_inff() && mj != -__builtin_inff()) ? exp2f(mj - M) : 0.0f;
    lsc[lane] = jl < ns ? ml.y : 0.0f;
  }
  __syncthreads();
  float den = 0.0f, o = 0.0f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float sc = wsc[j];
      den = fmaf(lsc[j], sc, den);
      o = fmaf(a[j], sc, o);
    }
    if (s2 != -__builtin_inff()) den += exp2f(s2 - M);
  }
  if (lane < 32) {
    const float r = den > 0.0f ? o / den : 0.0f;
    const size_t ob = ((size_t)t * kHq + hh) * kD + d0 + lane;
    if (p.out_f32) static_cast<float*>(p.out)[ob] = r;
    else static_cast<uint16_t*>(p.out)[ob] = f32_to_bf16(r);
  }
}

size_t attn_workspace_bytes(int T, int nsplit) {
  return (size_t)T * nsplit * kHq * kPartStride * sizeof(float);
}

// DSA lists (k up to 2048) split in 64-row pieces (enough workgroups to fill the chip);
// a sliding window of up to 128 rows runs in one workgroup per token (no merge).
constexpr int kSwaRows = 128;
int attn_splits(int mode, int list_len) {
  const int rows = mode == 0 ? kSplitRows : kSwaRows;
  return (list_len + rows - 1) / rows;
}

hipError_t launch_attention(int mode, int kvdt, const void* q, const void* kc, const void* vc,
                            const float* ks, const float* vs, const int32_t* idx, int k, int T,
                            int64_t L, int64_t ring_cap, int64_t pos0, int window, float sm_scale,
                            const float* sink, void* out, int out_f32, void* ws, int num_cu,
                            hipStream_t st) {
  AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kc = static_cast<const uint8_t*>(kc);
  p.vc = static_cast<const uint8_t*>(vc);
  p.ks = ks;
  p.vs = vs;
  p.idx = idx;
  p.k = k;
  p.T = T;
  p.L = L;
  p.ring_cap = ring_cap;
  p.pos0 = pos0;
  p.window = window;
  p.sm_log2 = sm_scale * 1.4426950408889634f;
  p.sink = sink;
  p.out = out;
  p.out_f32 = out_f32;
  p.nsplit = attn_splits(mode, mode == 0 ? k : window);
  p.part = static_cast<float*>(ws);
#ifdef DSA_TRACE
  p.trace = dsa_trace_buffer() ? dsa_trace_buffer() + 768 * 16 : nullptr;   // rows 768.. of the buffer
#endif
  (void)num_cu;
  const dim3 grid(p.nsplit, T);
  if (mode == 0) {
    // 512 threads: twice the staging loads in flight per workgroup
    if (kvdt == 0) hipLaunchKernelGGL((attn_kernel<0, 0, kSplitRows, 2 * kAttnThreads>), grid, dim3(2 * kAttnThreads), 0, st, p);
    else hipLaunchKernelGGL((attn_kernel<1, 0, kSplitRows, 2 * kAttnThreads>), grid, dim3(2 * kAttnThreads), 0, st, p);
  } else {
    if (kvdt == 0) hipLaunchKernelGGL((attn_kernel<0, 1, kSwaRows, 4 * kAttnThreads>), grid, dim3(4 * kAttnThreads), 0, st, p);
    else hipLaunchKernelGGL((attn_kernel<1, 1, kSwaRows, 4 * kAttnThreads>), grid, dim3(4 * kAttnThreads), 0, st, p);
  }
  if (p.nsplit > 1) {
#ifdef DSA_TRACE
    p.trace = nullptr;
#endif
    hipLaunchKernelGGL(attn_merge_kernel, dim3(32, T), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace dsa
