// C ABI of the DSA decode/verify step (declarations and contracts in include/dsa.h):
// host-side argument validation, workspace layout and kernel dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/dsa.h"
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace {

thread_local char g_err[512] = "";

dsa_status_t hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return e == hipErrorCooperativeLaunchTooLarge ? DSA_ERR_LAUNCH : DSA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// CUs the launch geometry is cut for.  Test hook: the environment variable DSA_NUM_CU,
// when set to a positive number below the device's count, stands in for a device with that
// many CUs (the selection then cuts the context into fewer, longer chunks; residency is
// still checked against the real device).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  if (const char* h = getenv("DSA_NUM_CU")) {
    const long v = strtol(h, nullptr, 10);
    if (v > 0 && v < n) n = (int)v;
  }
  return n;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int64_t kMaxL = 0x7fffffffLL;

dsa_status_t check_block(int T, int64_t L, int64_t pos0) {
  if (T < 1 || T > dsa::kMaxT) return DSA_ERR_SHAPE;
  if (pos0 < 0 || L < 1 || L > kMaxL || pos0 + T > L) return DSA_ERR_SHAPE;
  return DSA_OK;
}

__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---- layer-step workspace layout.  Every workspace starts with the control block
// (dsa::ctl); in a layer workspace the projection's counter and the selection's launch
// counter, error word and tau slots share it.
struct LayerWs {
  size_t proj, q_att, q_idx, w_idx, attn_out, idx, attn, tags, sel, total;
};

LayerWs layer_ws(int kind, int T, int64_t L, int k, int window, int ncu) {
  LayerWs w{};
  size_t o = 0;
  w.proj = o; o = align_up(o + dsa::proj_workspace_bytes());     // control block + k_I staging
  w.q_att = o; o = align_up(o + (size_t)dsa::kMaxT * dsa::kHq * dsa::kD * 2);
  w.q_idx = o; o = align_up(o + (size_t)dsa::kMaxT * dsa::kHI * dsa::kDI * 2);
  w.w_idx = o; o = align_up(o + (size_t)dsa::kMaxT * dsa::kHI * 4);
  w.attn_out = o; o = align_up(o + (size_t)dsa::kMaxT * dsa::kHq * dsa::kD * 2);
  const int list = kind == DSA_LAYER_DSA ? k : window;
  w.idx = o; o = align_up(o + (kind == DSA_LAYER_DSA ? (size_t)dsa::kMaxT * k * 4 : 0));
  w.attn = o; o = align_up(o + dsa::attn_workspace_bytes(dsa::kMaxT, dsa::attn_splits(kind == DSA_LAYER_DSA ? 0 : 1, list)));
  w.tags = o; o = align_up(o + (kind == DSA_LAYER_DSA ? dsa::layer_tail_tag_bytes(k) : 0));
  w.sel = o;
  if (kind == DSA_LAYER_DSA) o = align_up(o + dsa::select_data_bytes(T, L, k, ncu));
  w.total = o;
  return w;
}

// Checks of one layer's configuration, weights and cache for a block of T tokens at pos0
// (shared by the layer step and the module step).
dsa_status_t check_layer(const dsa_layer_config_t* cfg, const dsa_layer_weights_t* w,
                         const dsa_layer_cache_t* cache, int T, int64_t pos0, int ncu) {
  if (!cfg || !w || !cache) return DSA_ERR_NULL;
  if (!w->rms_gamma || !w->w_qkvi || !w->w_o || !cache->k || !cache->v) return DSA_ERR_NULL;
  if (w->w_dtype != DSA_BF16 && w->w_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  const bool w8a8 = w->w_dtype == DSA_FP8_E4M3;
  if (w8a8 != (w->w_qkvi_scale != nullptr) || w8a8 != (w->w_o_scale != nullptr)) return DSA_ERR_DTYPE;
  const bool dsa_kind = cfg->kind == DSA_LAYER_DSA;
  if (!dsa_kind && cfg->kind != DSA_LAYER_SWA) return DSA_ERR_SHAPE;
  if (dsa_kind && (!cache->k_idx || !cache->k_idx_scale)) return DSA_ERR_NULL;
  if (cfg->hidden != dsa::kHidden) return DSA_ERR_SHAPE;
  if (T < 1 || T > dsa::kMaxT || pos0 < 0) return DSA_ERR_SHAPE;
  const int64_t L = pos0 + T;
  if (dsa_kind) {
    if (cfg->top_k < 1 || cfg->top_k > dsa::kMaxTopK) return DSA_ERR_SHAPE;
    if (L > cache->capacity || L > dsa::select_max_context(ncu)) return DSA_ERR_SHAPE;
  } else {
    if (cfg->window < 1 || cfg->window > dsa::kMaxTopK) return DSA_ERR_SHAPE;
    if (cache->capacity < (int64_t)cfg->window + T - 1 || cache->capacity > kMaxL) return DSA_ERR_SHAPE;
  }
  if (!aligned16(w->rms_gamma) || !aligned16(w->w_qkvi) || !aligned16(w->w_o) || !aligned16(cache->k) ||
      !aligned16(cache->v) || (cache->k_idx && !aligned16(cache->k_idx)) || (cfg->sink && !aligned16(cfg->sink)))
    return DSA_ERR_ALIGN;
  return DSA_OK;
}

// ---- module-step workspace: the SWA chain's region (its own control block), two layer
// outputs between launches, and a layer-step workspace for the layers that run one by one
struct ModuleWs {
  size_t chain, xa, xb, layer, layer_bytes, total;
};

ModuleWs module_ws(int T, int64_t L, int k, int ncu) {
  ModuleWs m{};
  size_t o = 0;
  m.chain = o; o = align_up(o + dsa::swa_chain_workspace_bytes());
  m.xa = o; o = align_up(o + (size_t)dsa::kMaxT * dsa::kHidden * 2);
  m.xb = o; o = align_up(o + (size_t)dsa::kMaxT * dsa::kHidden * 2);
  m.layer = o;
  size_t lb = layer_ws(DSA_LAYER_SWA, T, L, 0, dsa::kMaxTopK, ncu).total;
  if (k > 0) {
    const size_t ld = layer_ws(DSA_LAYER_DSA, T, L, k, 0, ncu).total;
    lb = ld > lb ? ld : lb;
  }
  m.layer_bytes = lb;
  m.total = align_up(o + lb);
  return m;
}

// Layer i joins an SWA chain that starts at layer c: bf16 weights, the same window,
// norm, rotary and softmax constants and ring capacity, and a window that fits one
// workgroup.
bool chains_with(const dsa_layer_config_t* cfg, const dsa_layer_weights_t* w, const dsa_layer_cache_t* cache,
                 int i, int c, int T) {
  const dsa_layer_config_t& a = cfg[i];
  const dsa_layer_config_t& z = cfg[c];
  return a.kind == DSA_LAYER_SWA && w[i].w_dtype == DSA_BF16 && dsa::swa_chain_fits(T, a.window) &&
         a.window == z.window && a.rms_eps == z.rms_eps && a.rope_theta == z.rope_theta &&
         a.sm_scale == z.sm_scale && cache[i].capacity == cache[c].capacity;
}


// ---- scratch of the allocation-free attention entry point: the split partials of the
// largest call (T = 8, k = 2048), one copy per GPU held until the process ends.  In host
// code `scratch` names a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)dsa::kMaxT * 32 * dsa::kHq * 132 * sizeof(float);   // 1,081,344
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (resolved on the first call on the device).
dsa_status_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "dsa_sparse_attn_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_err, sizeof(g_err), "dsa_sparse_attn_static: device %d beyond the %d supported", dev, kMaxDevices);
    return DSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                 "dsa_sparse_attn_static: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size is out of the supported range";
    case DSA_ERR_DTYPE: return "unsupported storage type";
    case DSA_ERR_ALIGN: return "a pointer or stride is not 16-byte aligned";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_LAUNCH: return "launch shape cannot be co-resident on this device";
    case DSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* dsa_last_error(void) { return g_err; }

int64_t dsa_max_context(void) { return dsa::select_max_context(device_cus()); }

size_t dsa_workspace_bytes(int kind, int T, int64_t L, int k) {
  if (T < 1 || T > dsa::kMaxT || L < 1) return 0;
  const int ncu = device_cus();
  switch (kind) {
    case DSA_WS_TOPK:
    case DSA_WS_INDEX_TOPK:
      return dsa::select_workspace_bytes(T, L, k, ncu);
    case DSA_WS_SPARSE_ATTN:
      return dsa::ctl::kBytes + dsa::attn_workspace_bytes(T, dsa::attn_splits(0, k));
    case DSA_WS_SWA_ATTN:
      return dsa::ctl::kBytes + dsa::attn_workspace_bytes(T, dsa::attn_splits(1, k));
    case DSA_WS_LAYER_DSA:
      return layer_ws(DSA_LAYER_DSA, T, L, k, 0, ncu).total;
    case DSA_WS_LAYER_SWA:
      return layer_ws(DSA_LAYER_SWA, T, L, 0, k, ncu).total;
    case DSA_WS_MODULE:
      return module_ws(T, L, k, ncu).total;
  }
  return 0;
}

dsa_status_t dsa_workspace_status(const void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return DSA_ERR_NULL;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  if (ws_bytes < dsa::ctl::kBytes) return DSA_ERR_WORKSPACE;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dsa_workspace_status: stream synchronize");
  uint32_t word = 0;
  e = hipMemcpy(&word, static_cast<const uint32_t*>(ws) + dsa::ctl::kError, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "dsa_workspace_status: read of the error word");
  if (word != 0) {
    snprintf(g_err, sizeof(g_err),
             "a launch on this workspace gave up waiting for workgroups that were not resident; "
             "its outputs are not valid and the workspace must be cleared (dsa_workspace_init)");
    return DSA_ERR_LAUNCH;
  }
  return DSA_OK;
}

dsa_status_t dsa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return DSA_ERR_NULL;
  if (!aligned16(ws) || (ws_bytes & 15u)) return DSA_ERR_ALIGN;
  const size_t n16 = ws_bytes / 16;
  if (n16 == 0) return DSA_OK;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096)),
                     dim3(256), 0, (hipStream_t)stream, static_cast<uint4*>(ws), n16);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_workspace_init");
}

dsa_status_t dsa_indexer_scores(const void* q_idx, const float* w_idx, const void* k_idx,
                                const float* k_idx_scale, int k_dtype, int T, int64_t L,
                                int64_t pos0, float* scores, int64_t ld, void* stream) {
  if (!q_idx || !w_idx || !k_idx || !scores) return DSA_ERR_NULL;
  if (k_dtype != DSA_BF16 && k_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  if ((k_dtype == DSA_FP8_E4M3) != (k_idx_scale != nullptr)) return DSA_ERR_DTYPE;
  if (dsa_status_t s = check_block(T, L, pos0)) return s;
  if (ld < L || (ld & 3)) return DSA_ERR_SHAPE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(scores) || !aligned16(w_idx) ||
      (k_idx_scale && !aligned16(k_idx_scale)))
    return DSA_ERR_ALIGN;
  hipError_t e = dsa::launch_indexer_scores(q_idx, w_idx, k_idx, k_idx_scale, k_dtype == DSA_FP8_E4M3,
                                            T, L, pos0, scores, ld, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_indexer_scores");
}

static dsa_status_t check_topk_common(int T, int64_t L, int64_t pos0, int k, const int32_t* idx,
                                      void* ws, size_t ws_bytes, size_t* need) {
  if (!idx) return DSA_ERR_NULL;
  if (dsa_status_t s = check_block(T, L, pos0)) return s;
  if (k < 1 || k > dsa::kMaxTopK) return DSA_ERR_SHAPE;
  const int ncu = device_cus();
  if (L > dsa::select_max_context(ncu)) return DSA_ERR_SHAPE;
  *need = dsa::select_workspace_bytes(T, L, k, ncu);
  if (!ws || ws_bytes < *need) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws) || !aligned16(idx)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

dsa_status_t dsa_topk(const float* scores, int T, int64_t L, int64_t ld, int64_t pos0, int k,
                      int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  if (!scores) return DSA_ERR_NULL;
  if (ld < L || (ld & 3)) return DSA_ERR_SHAPE;
  if (!aligned16(scores)) return DSA_ERR_ALIGN;
  size_t need = 0;
  if (dsa_status_t s = check_topk_common(T, L, pos0, k, idx, ws, ws_bytes, &need)) return s;
  hipError_t e = dsa::launch_select(1, nullptr, nullptr, nullptr, nullptr, 0, scores, ld, T, L, pos0,
                                    k, idx, count, ws, static_cast<uint8_t*>(ws) + dsa::ctl::kBytes,
                                    device_cus(), (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_topk");
}

dsa_status_t dsa_index_topk(const void* q_idx, const float* w_idx, const void* k_idx,
                            const float* k_idx_scale, int k_dtype, int T, int64_t L,
                            int64_t pos0, int k, int32_t* idx, int32_t* count, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!q_idx || !w_idx || !k_idx) return DSA_ERR_NULL;
  if (k_dtype != DSA_BF16 && k_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  if ((k_dtype == DSA_FP8_E4M3) != (k_idx_scale != nullptr)) return DSA_ERR_DTYPE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx) ||
      (k_idx_scale && !aligned16(k_idx_scale)))
    return DSA_ERR_ALIGN;
  size_t need = 0;
  if (dsa_status_t s = check_topk_common(T, L, pos0, k, idx, ws, ws_bytes, &need)) return s;
  hipError_t e = dsa::launch_select(0, q_idx, w_idx, k_idx, k_idx_scale, k_dtype == DSA_FP8_E4M3, nullptr,
                                    0, T, L, pos0, k, idx, count, ws, static_cast<uint8_t*>(ws) + dsa::ctl::kBytes,
                                    device_cus(), (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_index_topk");
}

dsa_status_t dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, int kv_dtype,
                             const int32_t* idx, int k, int T, int64_t L, float sm_scale,
                             const float* sink, void* out, int out_dtype, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !idx || !out) return DSA_ERR_NULL;
  if (kv_dtype != DSA_BF16 && kv_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  const bool fp8 = kv_dtype == DSA_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return DSA_ERR_DTYPE;
  if (out_dtype != DSA_BF16 && out_dtype != DSA_FP32) return DSA_ERR_DTYPE;
  if (T < 1 || T > dsa::kMaxT || k < 1 || k > dsa::kMaxTopK || L < 1 || L > kMaxL) return DSA_ERR_SHAPE;
  const size_t need = dsa::ctl::kBytes + dsa::attn_workspace_bytes(T, dsa::attn_splits(0, k));
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(ws) ||
      (sink && !aligned16(sink)))
    return DSA_ERR_ALIGN;
  hipError_t e = dsa::launch_attention(0, fp8, q, k_cache, v_cache, k_scale, v_scale, idx, k, T, L, 0, 0, 0,
                                       sm_scale, sink, out, out_dtype == DSA_FP32,
                                       static_cast<uint8_t*>(ws) + dsa::ctl::kBytes, device_cus(),
                                       (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_sparse_attn");
}

dsa_status_t dsa_sparse_attn_static(const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale, int kv_dtype,
                                    const int32_t* idx, int k, int T, int64_t L, float sm_scale,
                                    const float* sink, void* out, int out_dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !idx || !out) return DSA_ERR_NULL;
  if (kv_dtype != DSA_BF16 && kv_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  const bool fp8 = kv_dtype == DSA_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return DSA_ERR_DTYPE;
  if (out_dtype != DSA_BF16 && out_dtype != DSA_FP32) return DSA_ERR_DTYPE;
  if (T < 1 || T > dsa::kMaxT || k < 1 || k > dsa::kMaxTopK || L < 1 || L > kMaxL) return DSA_ERR_SHAPE;
  const size_t need = dsa::attn_workspace_bytes(T, dsa::attn_splits(0, k));
  if (need > kStaticScratchBytes) {
    snprintf(g_err, sizeof(g_err), "dsa_sparse_attn_static: %zu scratch bytes needed, %zu available", need,
             kStaticScratchBytes);
    return DSA_ERR_WORKSPACE;
  }
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || (sink && !aligned16(sink)))
    return DSA_ERR_ALIGN;
  void* ptr = nullptr;
  if (dsa_status_t st = scratch_address(&ptr)) return st;
  // every split writes its whole partial before the merge reads it, so nothing in the
  // scratch has to start at zero
  hipError_t e = dsa::launch_attention(0, fp8, q, k_cache, v_cache, k_scale, v_scale, idx, k, T, L, 0, 0, 0,
                                       sm_scale, sink, out, out_dtype == DSA_FP32, ptr, device_cus(),
                                       (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_sparse_attn_static");
}

dsa_status_t swa_attn(const void* q, const void* k_ring, const void* v_ring, const float* k_scale,
                      const float* v_scale, int kv_dtype, int64_t ring_cap, int T, int64_t pos0,
                      int window, float sm_scale, const float* sink, void* out, int out_dtype,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k_ring || !v_ring || !out) return DSA_ERR_NULL;
  if (kv_dtype != DSA_BF16 && kv_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  const bool fp8 = kv_dtype == DSA_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return DSA_ERR_DTYPE;
  if (out_dtype != DSA_BF16 && out_dtype != DSA_FP32) return DSA_ERR_DTYPE;
  if (T < 1 || T > dsa::kMaxT || window < 1 || window > dsa::kMaxTopK || pos0 < 0) return DSA_ERR_SHAPE;
  if (ring_cap < (int64_t)window + T - 1 || ring_cap > kMaxL) return DSA_ERR_SHAPE;
  const size_t need = dsa::ctl::kBytes + dsa::attn_workspace_bytes(T, dsa::attn_splits(1, window));
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_ring) || !aligned16(v_ring) || !aligned16(out) || !aligned16(ws) ||
      (sink && !aligned16(sink)))
    return DSA_ERR_ALIGN;
  hipError_t e = dsa::launch_attention(1, fp8, q, k_ring, v_ring, k_scale, v_scale, nullptr, 0, T, 0, ring_cap,
                                       pos0, window, sm_scale, sink, out, out_dtype == DSA_FP32,
                                       static_cast<uint8_t*>(ws) + dsa::ctl::kBytes, device_cus(),
                                       (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "swa_attn");
}

dsa_status_t dsa_layer_step(const dsa_layer_config_t* cfg, const dsa_layer_weights_t* w,
                            const dsa_layer_cache_t* cache, const void* x_in, void* x_out,
                            int T, int64_t pos0, int32_t* idx_out, void* qkv_out, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!cfg || !w || !cache || !x_in || !x_out) return DSA_ERR_NULL;
  const int ncu = device_cus();
  if (dsa_status_t s = check_layer(cfg, w, cache, T, pos0, ncu)) return s;
  const bool w8a8 = w->w_dtype == DSA_FP8_E4M3;
  const float* wq_scale = w8a8 ? w->w_qkvi_scale : nullptr;
  const float* wo_scale = w8a8 ? w->w_o_scale : nullptr;
  const bool dsa_kind = cfg->kind == DSA_LAYER_DSA;
  if (x_in == x_out) return DSA_ERR_SHAPE;
  if (!dsa_kind && idx_out) return DSA_ERR_SHAPE;
  int64_t L = pos0 + T;
  const LayerWs lw = layer_ws(cfg->kind, T, L, cfg->top_k, cfg->window, ncu);
  if (!ws || ws_bytes < lw.total) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws) || !aligned16(x_in) || !aligned16(x_out) || (qkv_out && !aligned16(qkv_out)) ||
      (idx_out && !aligned16(idx_out)))
    return DSA_ERR_ALIGN;
  // The DSA layer runs as projection, selection, then separate attention, split-merge and
  // output-projection launches (five in all).  The environment variable
  // DSA_LAYER_PERSISTENT_TAIL=1 selects one persistent launch for everything after the
  // selection instead (three in all); it gives the same result bit for bit and measured
  // about 0.8 us slower per DSA layer on MI355X (0.9 us per module step), where a hand-off
  // between workgroups through memory costs about as much as a launch boundary.
  const char* pt = getenv("DSA_LAYER_PERSISTENT_TAIL");
  const bool fused = pt && pt[0] == '1';
  if (dsa_kind) {
    // nothing is launched (and no cache row written) unless the selection can run
    hipError_t e0 = dsa::select_check_resident(0, 1, T, L, pos0, cfg->top_k, ncu);
    if (e0 == hipSuccess && fused) e0 = dsa::attn_oproj_check_resident(w8a8, ncu);
    if (e0 != hipSuccess) return hip_fail(e0, "dsa_layer_step: workgroups cannot all be resident");
  }
  hipStream_t st = (hipStream_t)stream;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  void* q_att = w8 + lw.q_att;
  void* q_idx = w8 + lw.q_idx;
  float* w_idx = reinterpret_cast<float*>(w8 + lw.w_idx);
  void* attn_out = w8 + lw.attn_out;
  hipError_t e = dsa::launch_proj_qkv(dsa_kind ? 0 : 1, x_in, w->rms_gamma, w->w_qkvi, wq_scale, T, cfg->rms_eps,
                                      cfg->rope_theta, pos0, qkv_out, q_att, q_idx, w_idx, cache->k,
                                      cache->v, dsa_kind ? 0 : cache->capacity, cache->k_idx,
                                      cache->k_idx_scale, w8 + lw.proj, st);
  if (e != hipSuccess) return hip_fail(e, "dsa_layer_step: projection");
  if (dsa_kind && fused) {
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(w8 + lw.idx);
    e = dsa::launch_select(0, q_idx, w_idx, cache->k_idx, cache->k_idx_scale, 1, nullptr, 0, T, L, pos0,
                           cfg->top_k, idx, nullptr, w8, w8 + lw.sel, ncu, st);
    if (e != hipSuccess) return hip_fail(e, "dsa_layer_step: index/top-k");
    e = dsa::launch_attn_oproj(idx, T, L, cfg->top_k, w8, q_att, cache->k, cache->v, cfg->sm_scale, cfg->sink,
                               w8 + lw.tags, w->w_o, wo_scale, x_in, x_out, ncu, st);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_layer_step: attention + output projection");
  }
  if (dsa_kind) {
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(w8 + lw.idx);
    e = dsa::launch_select(0, q_idx, w_idx, cache->k_idx, cache->k_idx_scale, 1, nullptr, 0, T, L, pos0,
                           cfg->top_k, idx, nullptr, w8, w8 + lw.sel, ncu, st);
    if (e != hipSuccess) return hip_fail(e, "dsa_layer_step: index/top-k");
    e = dsa::launch_attention(0, 0, q_att, cache->k, cache->v, nullptr, nullptr, idx, cfg->top_k, T, L, 0, 0,
                              0, cfg->sm_scale, cfg->sink, attn_out, 0, w8 + lw.attn, ncu, st);
  } else {
    if (dsa::swa_out_fits(T, cfg->window)) {
      // the window is small enough for every output-projection workgroup to recompute it
      e = dsa::launch_swa_out(q_att, cache->k, cache->v, cache->capacity, pos0, T, cfg->window, cfg->sm_scale,
                              cfg->sink, w->w_o, wo_scale, x_in, x_out, st);
      return e == hipSuccess ? DSA_OK : hip_fail(e, "dsa_layer_step: window attention + output projection");
    }
    e = dsa::launch_attention(1, 0, q_att, cache->k, cache->v, nullptr, nullptr, nullptr, 0, T, 0,
                              cache->capacity, pos0, cfg->window, cfg->sm_scale, cfg->sink, attn_out, 0,
                              w8 + lw.attn, ncu, st);
  }
  if (e != hipSuccess) return hip_fail(e, "dsa_layer_step: attention");
  e = dsa::launch_proj_out(attn_out, w->w_o, wo_scale, x_in, x_out, T, w8 + lw.proj, st);
  if (e != hipSuccess) return hip_fail(e, "dsa_layer_step: output projection");
  return DSA_OK;
}

dsa_status_t dsa_module_step(int n_layers, const dsa_layer_config_t* cfg, const dsa_layer_weights_t* w,
                             const dsa_layer_cache_t* cache, const void* x_in, void* x_out, int T, int64_t pos0,
                             int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  if (!cfg || !w || !cache || !x_in || !x_out) return DSA_ERR_NULL;
  if (n_layers < 1 || n_layers > DSA_MAX_MODULE_LAYERS) return DSA_ERR_SHAPE;
  if (x_in == x_out) return DSA_ERR_SHAPE;
  const int ncu = device_cus();
  int kmax = 0, last_dsa = -1;
  for (int i = 0; i < n_layers; ++i) {
    if (dsa_status_t s = check_layer(&cfg[i], &w[i], &cache[i], T, pos0, ncu)) return s;
    if (cfg[i].kind == DSA_LAYER_DSA) {
      kmax = cfg[i].top_k > kmax ? cfg[i].top_k : kmax;
      last_dsa = i;
    }
  }
  if (idx_out && last_dsa < 0) return DSA_ERR_SHAPE;
  const int64_t L = pos0 + T;
  const ModuleWs mw = module_ws(T, L, kmax, ncu);
  if (!ws || ws_bytes < mw.total) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws) || !aligned16(x_in) || !aligned16(x_out) || (idx_out && !aligned16(idx_out)))
    return DSA_ERR_ALIGN;
  // nothing is launched (and no cache row written) unless every selection can run
  for (int i = 0; i < n_layers; ++i)
    if (cfg[i].kind == DSA_LAYER_DSA) {
      hipError_t e = dsa::select_check_resident(0, 1, T, L, pos0, cfg[i].top_k, ncu);
      if (e != hipSuccess) return hip_fail(e, "dsa_module_step: workgroups cannot all be resident");
    }
  // Layers run one layer step after another, all enqueued on the stream with nothing
  // between them on the host.  With DSA_MODULE_CHAIN=1 consecutive SWA layers run as one
  // persistent launch instead (when its workgroups can all be resident): the same bits,
  // but measured slower on MI355X (five SWA layers at 2^20 positions: 94 us against
  // 67 us), because handing each layer's output to every projecting workgroup through
  // memory costs more than a launch boundary.
  const char* ch = getenv("DSA_MODULE_CHAIN");
  const bool chain = ch && ch[0] == '1' && dsa::swa_chain_check_resident(ncu) == hipSuccess;
  (void)hipGetLastError();
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  void* buf[2] = {w8 + mw.xa, w8 + mw.xb};
  hipStream_t st = (hipStream_t)stream;
  const void* cur = x_in;
  int sel = 0;
  for (int i = 0; i < n_layers;) {
    int j = i + 1;
    if (chain && chains_with(cfg, w, cache, i, i, T))
      while (j < n_layers && j - i < dsa::kMaxChain && chains_with(cfg, w, cache, j, i, T)) ++j;
    void* out = j == n_layers ? x_out : buf[sel];
    if (chain && chains_with(cfg, w, cache, i, i, T)) {
      dsa::SwaChainLayer ls[dsa::kMaxChain];
      for (int q = i; q < j; ++q)
        ls[q - i] = dsa::SwaChainLayer{w[q].rms_gamma, w[q].w_qkvi, w[q].w_o, cache[q].k, cache[q].v, cfg[q].sink};
      hipError_t e = dsa::launch_swa_chain(j - i, ls, cur, out, T, pos0, cfg[i].window, cfg[i].sm_scale,
                                           cfg[i].rms_eps, cfg[i].rope_theta, cache[i].capacity, w8 + mw.chain, ncu,
                                           st);
      if (e != hipSuccess) return hip_fail(e, "dsa_module_step: SWA layers");
    } else {
      if (dsa_status_t s = dsa_layer_step(&cfg[i], &w[i], &cache[i], cur, out, T, pos0,
                                          i == last_dsa ? idx_out : nullptr, nullptr, w8 + mw.layer,
                                          mw.layer_bytes, stream))
        return s;
    }
    cur = out;
    sel ^= 1;
    i = j;
  }
  return DSA_OK;
}

}  // extern "C"
