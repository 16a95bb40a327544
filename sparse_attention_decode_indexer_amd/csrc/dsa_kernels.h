// Host-side launchers of the gfx950 kernels (called by the C ABI in capi.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "select_geometry.h"

namespace dsa {


hipError_t launch_indexer_scores(const void* q_idx, const float* w_idx, const void* k_idx,
                                 const float* k_scale, int kdt, int T, int64_t L, int64_t pos0,
                                 float* scores, int64_t ld, hipStream_t st);

size_t select_workspace_bytes(int T, int64_t L, int k, int num_cu);   // control block + data
size_t select_data_bytes(int T, int64_t L, int k, int num_cu);
// hipErrorCooperativeLaunchTooLarge when the selection's workgroups cannot all be resident
hipError_t select_check_resident(int src, int kdt, int T, int64_t L, int64_t pos0, int k, int num_cu);
hipError_t resident_capacity(const void* fn, int threads, int num_cu, int64_t* cap);
// src 0: scan k_idx (fused); src 1: read scores.  ctl: the workspace's control block;
// data: select_data_bytes of slots and candidate lists
hipError_t launch_select(int src, const void* q_idx, const float* w_idx, const void* k_idx,
                         const float* k_scale, int kdt, const float* scores, int64_t ld, int T,
                         int64_t L, int64_t pos0, int k, int32_t* idx, int32_t* count, void* ctl,
                         void* data, int num_cu, hipStream_t st);

// The DSA layer after its selection as one persistent launch of num_cu workgroups
// (attention over idx, split merge, output projection + residual): ctl = the workspace's
// control block (the selection's launch counter gives the tag), tags =
// layer_tail_tag_bytes(k) of tagged hand-off words.  w_o_scale != nullptr selects W8A8.
size_t layer_tail_tag_bytes(int k);
hipError_t launch_attn_oproj(const int32_t* idx, int T, int64_t L, int k, void* ctl, const void* q_att,
                             const void* kcache, const void* vcache, float sm_scale, const float* sink, void* tags,
                             const void* w_o, const float* w_o_scale, const void* x, void* xout, int num_cu,
                             hipStream_t st);
hipError_t attn_oproj_check_resident(bool w8a8, int num_cu);

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

// A run of up to kMaxChain consecutive SWA layers (bf16 weights, one window, W + T - 1 <=
// 160) as one persistent launch of 256 workgroups; ws: swa_chain_workspace_bytes(), its
// control block first.  hipErrorCooperativeLaunchTooLarge when the workgroups cannot all
// be resident.
constexpr int kMaxChain = 8;
struct SwaChainLayer {
  const void* gamma;
  const void* w_qkv;
  const void* w_o;
  void* kring;
  void* vring;
  const float* sink;
};
size_t swa_chain_workspace_bytes();
bool swa_chain_fits(int T, int window);
hipError_t swa_chain_check_resident(int num_cu);
hipError_t launch_swa_chain(int n, const SwaChainLayer* layers, const void* x_in, void* x_out, int T,
                            int64_t pos0, int window, float sm_scale, float eps, float theta, int64_t ring_cap,
                            void* ws, int num_cu, hipStream_t st);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

#ifdef DSA_TRACE
uint64_t* dsa_trace_buffer();   // profiling builds: phase-timestamp buffer (or null)
#endif

}  // namespace dsa
