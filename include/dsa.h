/*
 * dsa.h -- C ABI of a single-GPU decode/verify step of a DeepSeek-Sparse-Attention
 * (DSA) layer and its sliding-window (SWA) sibling, for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research).
 *   - §Model Architecture: a lightweight indexer scores the full history while the
 *     backbone attends only a selected subset of positions; the full KV cache is kept.
 *   - §Hybrid SWA-DSA Architecture: DSA keeps the top 2,048 positions, SWA a 128-token
 *     window; GQA with four KV groups; a 16-head indexer; both attention types carry a
 *     sink bias.
 *   - §A DSA layer: from 29 kernels to one: the stage list of one layer step (input
 *     RMSNorm, Q/K/V projections, RoPE, KV-cache writes, indexer GEMM, top-k selection,
 *     sparse gathering, attention, output projection).
 *   - §Optimizing inside the kernel: weights are fetched while RMSNorm runs; selected
 *     K/V rows are staged on chip split by split; eight query heads per GPU.
 *   - §GPU Memory Optimization: top-k indices are kept as an explicit result.
 *   - §Why single-stream speed matters for RL: results are bitwise deterministic.
 *
 * Shapes of one GPU's share (fixed in this version):
 *   H_q = 8 query heads sharing one KV head, head width D = 128,
 *   indexer: H_I = 16 heads of width D_I = 64, T (verify block) in [1, 8].
 *
 * Conventions
 *   - Every tensor argument is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or synchronises; scratch lives in a caller workspace whose size
 *     dsa_workspace_bytes() returns.
 *   - bf16 is IEEE bfloat16 stored as uint16; fp8 is OCP FP8 e4m3fn (bias 7, no
 *     infinities, max 448) with one fp32 scale per cache row: value = scale * code.
 *   - Rows are contiguous and row-major; row strides equal the row width unless stated.
 *   - Positions: the block's T new tokens sit at positions pos0 .. pos0+T-1; token t
 *     sees positions s <= pos0 + t (causal inside the block, itself included).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are stream-ordered,
 *     reentrant on distinct workspaces, and their outputs are a pure function of their
 *     inputs: the same inputs give bit-identical outputs.
 *   - Errors: arguments are checked on the host before anything is launched; on any
 *     error nothing is written and nothing is launched.  A failing HIP launch returns
 *     DSA_ERR_HIP (dsa_last_error() gives the message).  Faults inside a kernel surface
 *     at the caller's next synchronisation.
 *   - Workspaces: every workspace starts with a 16 KiB control block and must be
 *     zero-filled before its first use (allocate it with zeros or call
 *     dsa_workspace_init).  Its control words then carry state from call to call: the
 *     selection keeps a launch counter there (its slots are tagged with the counter, so
 *     no call has to clear them), and every call that completes leaves the words valid
 *     for the next one, so one workspace serves any number of stream-ordered calls,
 *     including replays of a captured graph.  Two calls that may run at the same time
 *     need distinct workspaces; a workspace must not be copied or re-zeroed while calls
 *     that use it are in flight.
 *   - Co-residency: the selection (dsa_topk, dsa_index_topk, the DSA layer step) runs
 *     one launch whose workgroups hand data to each other, so all of them must be
 *     resident at once.  The call checks on the host that the device can hold them and
 *     returns DSA_ERR_LAUNCH otherwise, before anything is launched.  Kernels of other
 *     streams or processes that occupy compute units at the same time can still keep a
 *     workgroup from starting; every wait inside the launch is bounded (0.2 s), and a
 *     wait that gives up sets a sticky error word in the workspace and writes an empty
 *     selection (indices -1, count 0) for the tokens it concerns.  dsa_workspace_status
 *     reports it; while the word is set, later selection calls on that workspace write
 *     empty selections and nothing else, until dsa_workspace_init clears it.
 *     (Test hook: the environment variable DSA_RESIDENT_LIMIT=n makes the host check
 *     assume at most n resident workgroups.)
 *   - Context length.  The selection cuts [0, L) into one chunk per compute unit.  Up to
 *     4096 keys per chunk every score stays on chip; longer chunks (up to 65536 keys)
 *     keep the scores past the first 4096 in the workspace, whose size
 *     (dsa_workspace_bytes) grows by 32 bytes per such key.  The selection is the same
 *     either way.  (Test hook: the environment variable DSA_NUM_CU=n, n below the
 *     device's count, cuts the geometry for n compute units; workspaces must then be
 *     sized with the same setting.)
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,      /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,     /* a size is out of the supported range */
  DSA_ERR_DTYPE = 3,     /* unsupported storage type for this argument */
  DSA_ERR_ALIGN = 4,     /* a pointer or stride is not 16-byte aligned */
  DSA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than dsa_workspace_bytes() */
  DSA_ERR_LAUNCH = 6,    /* the launch shape cannot be co-resident on this device */
  DSA_ERR_HIP = 7        /* a HIP runtime call failed */
} dsa_status_t;

typedef enum { DSA_BF16 = 0, DSA_FP8_E4M3 = 1, DSA_FP32 = 2 } dsa_dtype_t;

/* which call a workspace is sized for */
typedef enum {
  DSA_WS_TOPK = 1,        /* dsa_topk */
  DSA_WS_INDEX_TOPK = 2,  /* dsa_index_topk */
  DSA_WS_SPARSE_ATTN = 3, /* dsa_sparse_attn */
  DSA_WS_SWA_ATTN = 4,    /* swa_attn */
  DSA_WS_LAYER_DSA = 5,   /* dsa_layer_step, kind = DSA */
  DSA_WS_LAYER_SWA = 6,   /* dsa_layer_step, kind = SWA */
  DSA_WS_MODULE = 7       /* dsa_module_step; k = largest top_k of its DSA layers (0: none) */
} dsa_ws_kind_t;

/*
 * Indexer scores (§Model Architecture: the indexer scores the full history).
 *
 *   scores[t][s] = sum_h w_idx[t][h] * relu(q_idx[t][h] . k_idx[s]) * k_scale[s]
 *   for s <= pos0 + t;  scores[t][s] = -INFINITY for pos0 + t < s < L.
 *
 * q_idx   [T][16][64] bf16.   w_idx [T][16] fp32 (any sign).
 * k_idx   [L][64] bf16 (k_dtype = DSA_BF16, k_idx_scale must be NULL) or
 *         [L][64] e4m3 codes with k_idx_scale [L] fp32 > 0 (k_dtype = DSA_FP8_E4M3).
 * scores  [T][ld] fp32, ld >= L, ld % 4 == 0; columns >= L are not written.
 * 1 <= T <= 8, pos0 >= 0, pos0 + T <= L < 2^31.
 * Accumulation is fp32 in a fixed order; the same code computes the scores inside
 * dsa_index_topk, so both calls produce bit-identical scores.
 */
dsa_status_t dsa_indexer_scores(const void* q_idx, const float* w_idx, const void* k_idx,
                                const float* k_idx_scale, int k_dtype, int T, int64_t L,
                                int64_t pos0, float* scores, int64_t ld, void* stream);

/*
 * Top-k selection (§Hybrid SWA-DSA Architecture: the top 2,048 positions; §GPU Memory
 * Optimization: the indices are kept).
 *
 * For each token t, among the visible positions s <= pos0 + t, selects the
 * k_eff = min(k, pos0 + t + 1) positions ranked first by (score descending, position
 * ascending) -- ties go to the lower position, -0 equals +0.  Writes them to
 * idx[t][0 .. k_eff) in ascending position order and -1 to idx[t][k_eff .. k);
 * count[t] = k_eff when count is not NULL.  Scores must not be NaN.
 *
 * scores [T][ld] fp32 (as written by dsa_indexer_scores), 1 <= k <= 2048,
 * 1 <= T <= 8, pos0 + T <= L <= dsa_max_context(), ld >= L, ld % 4 == 0.
 * idx [T][k] int32, count [T] int32 or NULL.  ws: DSA_WS_TOPK.
 */
dsa_status_t dsa_topk(const float* scores, int T, int64_t L, int64_t ld, int64_t pos0, int k,
                      int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/*
 * Indexer scan fused with top-k: the result of dsa_indexer_scores followed by dsa_topk,
 * bit for bit, without writing the score matrix to memory (scores stay on chip).
 * Arguments as in those two calls.  ws: DSA_WS_INDEX_TOPK.
 */
dsa_status_t dsa_index_topk(const void* q_idx, const float* w_idx, const void* k_idx,
                            const float* k_idx_scale, int k_dtype, int T, int64_t L,
                            int64_t pos0, int k, int32_t* idx, int32_t* count, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Sparse GQA attention over selected rows (§Model Architecture: attention over the
 * selected subset only; §Hybrid SWA-DSA Architecture: GQA, sink bias; §Optimizing
 * inside the kernel: selected K/V rows staged on chip split by split).
 *
 * For token t and query head h, over the list J = {idx[t][j] : 0 <= idx[t][j] < L}
 * (entries outside [0, L) are skipped; duplicates count once per entry):
 *   z_j = sm_scale * q[t][h] . K[j],   m = max(max_j z_j, sink[h])
 *   out[t][h] = sum_j e^(z_j - m) V[j] / (sum_j e^(z_j - m) + e^(sink[h] - m))
 * without the sink terms when sink is NULL; an empty J gives 0.
 *
 * q [T][8][128] bf16.  k_cache, v_cache [L][128] bf16, or e4m3 codes with
 * k_scale, v_scale [L] fp32 (kv_dtype = DSA_FP8_E4M3; must be NULL for bf16).
 * idx [T][k] int32, 1 <= k <= 2048.  sink [8] fp32 logits or NULL.
 * out [T][8][128], out_dtype DSA_BF16 or DSA_FP32.  ws: DSA_WS_SPARSE_ATTN.
 * Rows are processed in fixed splits of 64 list entries merged in split order.
 */
dsa_status_t dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, int kv_dtype,
                             const int32_t* idx, int k, int T, int64_t L, float sm_scale,
                             const float* sink, void* out, int out_dtype, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * dsa_sparse_attn without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, result and kernels as dsa_sparse_attn, minus ws / ws_bytes: the split
 * partials live in a library-owned device array of 1,081,344 bytes (the largest call,
 * T = 8, k = 2048), one per GPU, held until the process ends; a call needing more returns
 * DSA_ERR_WORKSPACE.  The call allocates nothing.  Every call on one GPU shares that
 * GPU's array, so calls that may overlap on one GPU (different streams, or concurrent
 * host threads) race and must not be issued; stream-ordered calls are safe.
 */
dsa_status_t dsa_sparse_attn_static(const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale, int kv_dtype,
                                    const int32_t* idx, int k, int T, int64_t L, float sm_scale,
                                    const float* sink, void* out, int out_dtype, void* stream);

/*
 * Sliding-window attention (§Hybrid SWA-DSA Architecture: a 128-token window; §Model
 * Architecture: per-token cost independent of context length).
 *
 * Token t at p = pos0 + t attends positions [max(0, p - window + 1), p], read from a
 * ring buffer where position p lives in slot p % ring_cap; the ring must hold all of
 * them, so ring_cap >= window + T - 1.  Same softmax and sink rule as dsa_sparse_attn.
 * q [T][8][128] bf16; k_ring, v_ring [ring_cap][128] bf16 (kv_dtype DSA_BF16, scales
 * NULL) or e4m3 codes with k_scale, v_scale [ring_cap] fp32 row scales (DSA_FP8_E4M3);
 * 1 <= window <= 2048.  out [T][8][128] bf16 or fp32.  ws: DSA_WS_SWA_ATTN.
 */
dsa_status_t swa_attn(const void* q, const void* k_ring, const void* v_ring, const float* k_scale,
                      const float* v_scale, int kv_dtype, int64_t ring_cap, int T, int64_t pos0,
                      int window, float sm_scale, const float* sink, void* out, int out_dtype,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * One layer step (§A DSA layer: from 29 kernels to one; §Optimizing inside the kernel).
 *
 * kind DSA:  y = RMSNorm(x_in) * gamma -> P = y . W_qkvi^T, P = [Q 1024 | K 128 | V 128 |
 *            q_I 1024 | k_I 64 | w_I 16] -> RoPE (rotate-half, theta) on Q, K, q_I, k_I at
 *            positions pos0 + t -> append K, V (bf16) and k_I (e4m3, per-row scale
 *            amax/448) at rows pos0 .. pos0+T-1 -> indexer over rows [0, pos0+T) ->
 *            top-k -> sparse attention -> x_out = x_in + O . W_o^T.
 * kind SWA:  P = [Q | K | V] -> RoPE on Q, K -> append K, V into the ring at slot p % cap
 *            -> window attention -> output projection + residual.
 * Rounding points: y, P, the rotated values and the attention output are rounded to
 * bf16; accumulation is fp32.
 *
 * Weights (out-features major), w_dtype DSA_BF16:
 *   rms_gamma [hidden] bf16; w_qkvi [N][hidden] bf16 with N = 2384 (DSA) or 1280 (SWA);
 *   w_o [hidden][1024] bf16; w_qkvi_scale, w_o_scale NULL.
 * W8A8 (w_dtype DSA_FP8_E4M3; §How it was built: W8A8 kernels were among those tuned;
 * §Get NaiveRT: the released checkpoint is W8A8): w_qkvi and w_o hold OCP e4m3fn codes in the
 * same layout, with one fp32 scale per weight row (w_qkvi_scale [N], w_o_scale [hidden]);
 * rms_gamma stays bf16.  Each projection input row (the normalised y, and the bf16
 * attention output before W_o) is quantised per token: amax = max |y|, scale =
 * fp32(amax / 448) and codes e4m3(fp32(y * fp32(448 / amax))) rounded to nearest even
 * (scale 1, codes 0 for an all-zero row); products of codes are accumulated in fp32 and
 * multiplied by both scales.
 * Cache (DSA): k, v [capacity][128] bf16; k_idx [capacity][64] e4m3; k_idx_scale
 *   [capacity] fp32; pos0 + T <= capacity, pos0 + T <= dsa_max_context().
 * Cache (SWA): k, v rings [capacity][128] bf16 holding positions
 *   [pos0 - window + 1, pos0); capacity >= window + T - 1; k_idx, k_idx_scale NULL.
 * x_in, x_out [T][hidden] bf16 (x_out must not alias x_in).  hidden = 4096.
 * idx_out [T][top_k] int32 (DSA only, optional): the selected positions.
 * qkv_out [T][N] bf16 (optional): the projection after RoPE.
 * ws: DSA_WS_LAYER_DSA or DSA_WS_LAYER_SWA sized for (T, pos0 + T, top_k).
 * A DSA layer runs as five stream-ordered launches (projection, index/top-k, attention,
 * split merge, output projection); with the environment variable
 * DSA_LAYER_PERSISTENT_TAIL=1 everything after the index/top-k runs as one persistent
 * launch instead, with the same result bit for bit.
 * --------------------------------------------------------------------------------- */
typedef enum { DSA_LAYER_DSA = 0, DSA_LAYER_SWA = 1 } dsa_layer_kind_t;

typedef struct {
  int kind;          /* dsa_layer_kind_t */
  int hidden;        /* 4096 */
  int top_k;         /* DSA: 1..2048 */
  int window;        /* SWA: 1..2048 */
  float rms_eps;     /* e.g. 1e-6 */
  float rope_theta;  /* e.g. 1e6 */
  float sm_scale;    /* e.g. 1/sqrt(128) */
  const float* sink; /* [8] fp32 or NULL */
} dsa_layer_config_t;

typedef struct {
  const void* rms_gamma;
  const void* w_qkvi;
  const void* w_o;
  int w_dtype;                /* DSA_BF16, or DSA_FP8_E4M3 for W8A8 */
  const float* w_qkvi_scale;  /* [N] fp32 (W8A8 only, else NULL) */
  const float* w_o_scale;     /* [hidden] fp32 (W8A8 only, else NULL) */
} dsa_layer_weights_t;

typedef struct {
  void* k;
  void* v;
  void* k_idx;
  float* k_idx_scale;
  int64_t capacity;
} dsa_layer_cache_t;

dsa_status_t dsa_layer_step(const dsa_layer_config_t* cfg, const dsa_layer_weights_t* w,
                            const dsa_layer_cache_t* cache, const void* x_in, void* x_out,
                            int T, int64_t pos0, int32_t* idx_out, void* qkv_out, void* ws,
                            size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ module step
 * §The execution model (naive.ai/en/research): the stages of the decode loop are fused
 * into larger kernels and the remaining boundaries are bridged on the device, without the
 * host in between.
 *
 * n_layers (1 .. DSA_MAX_MODULE_LAYERS) decoder layers applied in order to one block of T
 * tokens at pos0: layer i reads the output of layer i - 1 (x_in for layer 0) and the last
 * writes x_out; layer i computes what dsa_layer_step computes for cfg[i], w[i], cache[i],
 * and the result equals n_layers dsa_layer_step calls bit for bit.
 * The layers' launches are enqueued back to back with no host work between them (the
 * call can be captured into a HIP graph).  With DSA_MODULE_CHAIN=1 in the environment,
 * consecutive SWA layers with bf16 weights and the same window (window + T - 1 <= 160),
 * rms_eps, rope_theta, sm_scale and ring capacity run as ONE persistent launch per up to 8
 * layers instead: 256 workgroups, one per compute unit, all resident, that hand each
 * layer's Q/K/V and output to each other through launch-tagged words in the workspace
 * (when the device cannot hold them all at once, those layers run one layer step at a
 * time).  Both give the same bits; the persistent launch measured slower on MI355X.
 * idx_out [T][top_k] int32 (optional): the selection of the last DSA layer.
 * ws: DSA_WS_MODULE sized for (T, pos0 + T, largest top_k), zero-filled before first use;
 * like the other workspaces it carries launch counters and a sticky error word
 * (dsa_workspace_status).  Every argument is checked, and every selection's co-residency,
 * before anything is launched.
 * --------------------------------------------------------------------------------- */
#define DSA_MAX_MODULE_LAYERS 64

dsa_status_t dsa_module_step(int n_layers, const dsa_layer_config_t* cfg, const dsa_layer_weights_t* w,
                             const dsa_layer_cache_t* cache, const void* x_in, void* x_out, int T,
                             int64_t pos0, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------- helpers */

/* Bytes of workspace `kind` needs for T tokens, context length L and top-k k. */
size_t dsa_workspace_bytes(int kind, int T, int64_t L, int k);

/* Zero-fills a workspace on `stream` with a kernel (no hipMemset). */
dsa_status_t dsa_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Synchronises `stream`, then reads the workspace's sticky error word: DSA_OK, or
 * DSA_ERR_LAUNCH if a launch on the workspace gave up waiting for workgroups that were
 * not resident (its outputs are then not valid; dsa_last_error() says so).  The word
 * stays set until dsa_workspace_init.  Blocking; not for use under graph capture. */
dsa_status_t dsa_workspace_status(const void* ws, size_t ws_bytes, void* stream);

/* Largest context length L the top-k calls and dsa_layer_step accept on the current
 * device: 65536 positions per compute unit (16,777,216 on a 256-CU MI355X).  Past 4096
 * positions per compute unit (1,048,576 on MI355X) part of the scores is kept in the
 * workspace instead of on chip. */
int64_t dsa_max_context(void);

const char* dsa_status_string(dsa_status_t s);

/* Message of the last DSA_ERR_HIP / DSA_ERR_LAUNCH on this host thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
