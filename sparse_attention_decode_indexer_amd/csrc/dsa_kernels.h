// Host-side launchers of the gfx950 kernels (called by the C ABI in capi.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct SelGeometry {
  int chunk;    // keys per workgroup
  int nwg;      // workgroups
  int n_part;   // workgroups publishing a tau bound
  int m;        // tau rank (0: no bound)
  bool fits;    // chunk fits LDS and nwg fits the count arrays
};

hipError_t launch_indexer_scores(const void* q_idx, const float* w_idx, const void* k_idx,
                                 const float* k_scale, int kdt, int T, int64_t L, int64_t pos0,
                                 float* scores, int64_t ld, hipStream_t st);

SelGeometry select_geometry(int T, int64_t L, int64_t pos0, int k, int num_cu);
size_t select_workspace_bytes(int T, int64_t L, int k, int num_cu);
int64_t select_max_context(int num_cu);
// src 0: scan k_idx (fused); src 1: read scores
hipError_t launch_select(int src, const void* q_idx, const float* w_idx, const void* k_idx,
                         const float* k_scale, int kdt, const float* scores, int64_t ld, int T,
                         int64_t L, int64_t pos0, int k, int32_t* idx, int32_t* count, void* ws,
                         int num_cu, hipStream_t st);

size_t attn_workspace_bytes(int T, int nsplit);
int attn_splits(int mode, int list_len);   // mode 0: index list, 1: sliding window
// mode 0: sparse list idx; mode 1: sliding window over a ring
hipError_t launch_attention(int mode, int kvdt, const void* q, const void* kc, const void* vc,
                            const float* ks, const float* vs, const int32_t* idx, int k, int T,
                            int64_t L, int64_t ring_cap, int64_t pos0, int window, float sm_scale,
                            const float* sink, void* out, int out_f32, void* ws, int num_cu,
                            hipStream_t st);

size_t proj_workspace_bytes();
// wscale: per-row fp32 scales of e4m3 weights (W8A8), or nullptr for bf16 weights
hipError_t launch_proj_qkv(int kind, const void* x, const void* gamma, const void* w,
                           const float* wscale, int T, float eps, float theta, int64_t pos0,
                           void* qkv, void* q_att, void* q_idx, float* w_idx, void* kcache,
                           void* vcache, int64_t ring_cap, void* kidx, float* kidx_scale, void* ws,
                           hipStream_t st);
hipError_t launch_proj_out(const void* o, const void* w_o, const float* wscale, const void* x,
                           void* xout, int T, void* ws, hipStream_t st);

// sliding-window attention fused with the output projection (window + T - 1 <= 160 rows)
bool swa_out_fits(int T, int window);
hipError_t launch_swa_out(const void* q, const void* kring, const void* vring, int64_t ring_cap,
                          int64_t pos0, int T, int window, float sm_scale, const float* sink,
                          const void* w_o, const float* w_o_scale, const void* x, void* xout,
                          hipStream_t st);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

// streaming read of `bytes` (a multiple of 16) by `nblocks` workgroups; one word per
// workgroup into sink
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int nblocks, hipStream_t st);

#ifdef DSA_TRACE
uint64_t* dsa_trace_buffer();   // profiling builds: phase-timestamp buffer (or null)
#endif

}  // namespace dsa
