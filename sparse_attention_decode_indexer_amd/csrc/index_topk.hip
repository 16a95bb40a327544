// Indexer scan and exact top-k selection for gfx950.
//
// Method: NaiveAI, "Naive-N0.5-Flash: Building Frontier AI with AI", §Model Architecture
// (the indexer scores the full history, the backbone attends a selected subset) and
// §Hybrid SWA-DSA Architecture (16 indexer heads, top 2,048 positions).
//
// Score of key s for token t:  I[t,s] = sum_h w[t,h] * relu(q_I[t,h] . k[s]) (* row scale).
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16): one row tile = 2 tokens x 16 heads = 32 MFMA
// rows; the 32 MFMA columns are 32 consecutive keys; K = 64 indexer dims in 4 steps.
// A block of 8 tokens therefore fills 128 rows with no padding.  The epilogue does
// relu -> x w -> fixed-order head sum in registers (8 heads per lane, then one exchange
// with the lane 32 away) and, for e4m3 keys, one multiply by the row scale.
//
// Selection is one launch of one workgroup per chunk of C keys, all resident at once:
//   P1  scores of the chunk (computed, or read from memory) stay in LDS; each
//       workgroup derives a lower bound tau_wg of its m-th largest visible score from
//       per-group maxima and publishes min(tau) with an integer atomic;
//   P2  every workgroup writes its visible scores >= tau, in position order, as
//       (order key, position) candidates;
//   P3  the last workgroup to publish a token's candidates runs an exact radix select
//       over them and writes the selected positions in ascending order.
// P1 and P2 are separated by one grid barrier; inter-workgroup data moves only through
// agent-scope atomic loads/stores, so no cache writeback or invalidation is needed.
// Because at least m scores of each of n_part workgroups are >= tau and
// m * n_part >= k, the candidates always contain the k best; the result is exact and
// independent of tau.  All cross-workgroup arithmetic is integer, so the result is
// bitwise reproducible.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kTile = 32;        // keys per MFMA column tile
constexpr int kSelThreads = 256; // threads of the selection kernel
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kGroups = 32 * kSelWaves;   // score groups per workgroup and token
constexpr int kMaxChunk = 4096;  // keys per workgroup held in LDS
constexpr int kTauMaxM = 32;

// ----------------------------------------------------------------------------- tile math

template <int KDT>
struct KeyTile {
  uint4 raw[KDT == 0 ? 4 : 2];   // this lane's 32 dims of its key (bf16: 64 B, e4m3: 32 B)
  float scale;
};

// Lane l loads dims [32*(l>>5), +32) of key s0 + (l & 31); rows past L are clamped
// (their scores are masked by the caller).
template <int KDT>
DSA_DEV void load_key_tile(const uint8_t* __restrict__ kbase, const float* __restrict__ kscale,
                           int64_t L, int64_t s0, KeyTile<KDT>& kt) {
  const int l = threadIdx.x & 63;
  int64_t s = s0 + (l & 31);
  s = s < L ? s : L - 1;
  const int half = l >> 5;
  if constexpr (KDT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(kbase + s * 128 + half * 64);
    kt.raw[0] = p[0];
    kt.raw[1] = p[1];
    kt.raw[2] = p[2];
    kt.raw[3] = p[3];
    kt.scale = 1.0f;
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(kbase + s * 64 + half * 32);
    kt.raw[0] = p[0];
    kt.raw[1] = p[1];
    kt.scale = kscale[s];
  }
}

// A operands: row tile r, k-step j.  Lane l: row (l & 31) -> token 2r + ((l&31)>>4),
// head (l & 15); dims 32*(l>>5) + 8j .. +8 (the same dims the key operand uses).
template <int RT>
DSA_DEV void load_q_frags(const uint16_t* __restrict__ q_idx, int T, Frag8 (&qa)[RT][4]) {
  const int l = threadIdx.x & 63;
  const int half = l >> 5;
  const int row = l & 31;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int tt = 2 * r + (row >> 4);
    const int hh = row & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (tt < T) {
        qa[r][j].u = *reinterpret_cast<const uint4*>(q_idx + (tt * kHI + hh) * kDI + half * 32 + 8 * j);
      } else {
        qa[r][j].u = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
}

// Head weights for this lane's accumulator elements.  Element e of the 32x32 output
// holds row 8*(e>>2) + 4*half + (e&3): token 2r + (e>>3), head 8*((e>>2)&1) + 4*half + (e&3).
template <int RT>
DSA_DEV void load_w(const float* __restrict__ w_idx, int T, float (&wv)[RT][16]) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tt = 2 * r + (e >> 3);
      const int hh = 8 * ((e >> 2) & 1) + 4 * half + (e & 3);
      wv[r][e] = (tt < T) ? w_idx[tt * kHI + hh] : 0.0f;
    }
  }
}

// Scores of one 32-key tile: out[r] is the score of token 2r + (lane>>5) for key
// s0 + (lane & 31).  Fixed arithmetic order (the same in every kernel that calls it).
template <int KDT, int RT>
DSA_DEV void score_tile(const KeyTile<KDT>& kt, const Frag8 (&qa)[RT][4], const float (&wv)[RT][16],
                        float (&out)[RT]) {
  Frag8 kb[4];
  if constexpr (KDT == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j].u = kt.raw[j];
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&kt.raw[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[2 * j], 1.0f, false);
      bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[2 * j], 1.0f, true);
      bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[2 * j + 1], 1.0f, false);
      bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[2 * j + 1], 1.0f, true);
      kb[j].v = bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    }
  }
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    f32x16_t acc = {};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[r][j].v, kb[j].v, acc, 0, 0, 0);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) p0 = fmaf(wv[r][e], fmaxf(acc[e], 0.0f), p0);
#pragma unroll
    for (int e = 8; e < 16; ++e) p1 = fmaf(wv[r][e], fmaxf(acc[e], 0.0f), p1);
    const float send = half ? p0 : p1;
    const float recv = __shfl_xor(send, 32, 64);
    const float tot = (half ? p1 : p0) + recv;
    out[r] = (KDT == 1) ? tot * kt.scale : tot;
  }
}

// ----------------------------------------------------------------------------- scores kernel

constexpr int kScoreThreads = 256;
constexpr int kScoreTilesPerWave = 8;

template <int KDT, int RT>
__global__ void __launch_bounds__(kScoreThreads)
indexer_scores_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                      const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale,
                      int T, int64_t L, int64_t pos0, float* __restrict__ scores, int64_t ld) {
  Frag8 qa[RT][4];
  float wv[RT][16];
  load_q_frags<RT>(q_idx, T, qa);
  load_w<RT>(w_idx, T, wv);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int64_t ntiles = (L + kTile - 1) / kTile;
  const int64_t tile0 = ((int64_t)blockIdx.x * (kScoreThreads / 64) + wave) * kScoreTilesPerWave;
  KeyTile<KDT> cur, nxt;
  if (tile0 < ntiles) load_key_tile<KDT>(k_idx, k_scale, L, tile0 * kTile, cur);
  for (int i = 0; i < kScoreTilesPerWave; ++i) {
    const int64_t tile = tile0 + i;
    if (tile >= ntiles) break;
    if (i + 1 < kScoreTilesPerWave && tile + 1 < ntiles)
      load_key_tile<KDT>(k_idx, k_scale, L, (tile + 1) * kTile, nxt);
    float out[RT];
    score_tile<KDT, RT>(cur, qa, wv, out);
    const int64_t s = tile * kTile + (lane & 31);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int tt = 2 * r + half;
      if (tt < T && s < L) scores[tt * ld + s] = (s <= pos0 + tt) ? out[r] : -__builtin_inff();
    }
    cur = nxt;
  }
}

// ----------------------------------------------------------------------------- selection

struct SelParams {
  // score source
  const uint16_t* q_idx;
  const float* w_idx;
  const uint8_t* k_idx;
  const float* k_scale;
  const float* scores;   // materialised scores (SRC == 1)
  int64_t ld;
  // problem
  int T;
  int k;
  int64_t L;
  int64_t pos0;
  int chunk;             // keys per workgroup (multiple of 128, <= kMaxChunk)
  int nwg;               // workgroups (>= T)
  int m;                 // tau rank; 0 disables tau
  int n_part;            // workgroups [0, n_part) publish tau
  // outputs
  int32_t* idx;
  int32_t* count;
  // workspace
  uint32_t* ctl;         // control words (see namespace ctl)
  uint32_t* cnt;         // [T][nwg] candidate counts
  uint64_t* cand;        // [T][nwg][chunk] (position << 32 | order key)
};

struct SelShared {
  float sc[kMaxT][kMaxChunk];        // chunk scores (P1/P2); resolver scratch (P3)
  uint32_t gmax[kMaxT][kGroups];     // per-group maxima (order keys)
  uint32_t tau[kMaxT];
  uint32_t resolve[kMaxT];
  uint32_t scan[32];
};

// m-th largest of the kGroups group maxima of one token, computed by one wave.
DSA_DEV uint32_t mth_largest_wave(const uint32_t* g, int m) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = kGroups / 64;
  uint32_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = g[lane * PER + i];
  uint32_t cur = 0;
  for (int it = 0; it < m; ++it) {
    uint32_t mx = v[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) mx = max(mx, v[i]);
    cur = wave_max_u32(mx);
    // remove one occurrence (lowest lane, lowest slot)
    bool has = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) has |= (v[i] == cur);
    const uint64_t bal = __ballot(has);
    const int first = __builtin_ctzll(bal);
    if (lane == first) {
      bool done = false;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (!done && v[i] == cur) { v[i] = 0u; done = true; }
    }
  }
  return cur;
}

// Exact selection of the kk best candidates of token t.  Runs in one workgroup after
// every workgroup has published its candidates for t.
DSA_DEV void resolve_token(const SelParams& p, int t, SelShared& sh) {
  uint32_t* pre = reinterpret_cast<uint32_t*>(&sh.sc[0][0]);         // [nwg + 1]
  uint32_t* hist = pre + 1040;                                        // [2048]
  uint32_t* misc = hist + 2048;                                       // small
  const int tid = threadIdx.x;
  const int nwg = p.nwg;
  const uint32_t* cnt_t = p.cnt + (size_t)t * nwg;
  // prefix over workgroup counts
  uint32_t carry = 0;
  for (int base = 0; base < nwg; base += kSelThreads) {
    const int w = base + tid;
    const uint32_t c = (w < nwg) ? ald(cnt_t + w) : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kSelThreads>(c, sh.scan, &tot);
    if (w < nwg) pre[w] = carry + ex;
    carry += tot;
  }
  if (tid == 0) pre[nwg] = carry;
  __syncthreads();
  const uint32_t nc = carry;
  const int64_t vis = p.pos0 + t + 1;
  uint32_t kk = (uint32_t)((int64_t)p.k < vis ? p.k : vis);
  if (kk > nc) kk = nc;   // cannot happen when the bound holds; keeps reads in range
  const uint64_t* base = p.cand + (size_t)t * nwg * p.chunk;
  // contiguous run of candidates per thread, visited in position order
  const uint32_t run = (nc + kSelThreads - 1) / kSelThreads;
  const uint32_t g0 = min(nc, (uint32_t)tid * run);
  const uint32_t g1 = min(nc, g0 + run);
  auto visit = [&](auto&& fn) {
    if (g0 >= g1) return;
    int lo = 0, hi = nwg - 1;            // largest w with pre[w] <= g0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    int w = lo;
    uint32_t j = g0 - pre[w];
    for (uint32_t g = g0; g < g1; ++g) {
      while (g >= pre[w + 1]) { ++w; j = 0; }
      const uint64_t e = ald64(base + (size_t)w * p.chunk + j);
      fn((uint32_t)e, (uint32_t)(e >> 32));
      ++j;
    }
  };
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  visit([&](uint32_t key, uint32_t) { kmin = min(kmin, key); kmax = max(kmax, key); });
  kmin = block_min_u32<kSelThreads>(kmin, sh.scan);
  kmax = block_max_u32<kSelThreads>(kmax, sh.scan);
  uint32_t kstar;
  uint32_t take_eq;
  if (kk == nc) {
    kstar = kmin;
    take_eq = 0xffffffffu;
  } else {
    // MSB-first radix select on the bits where candidate keys differ
    const uint32_t diff = kmin ^ kmax;
    int hi = diff ? 32 - __builtin_clz(diff) : 0;
    uint32_t known = hi >= 32 ? 0u : (kmax & ~((1u << hi) - 1u));
    uint32_t need = kk;
    while (hi > 0) {
      const int dbits = hi < 11 ? hi : 11;
      const int lo = hi - dbits;
      const uint32_t nb = 1u << dbits;
      for (int b = tid; b < 2048; b += kSelThreads) hist[b] = 0u;
      __syncthreads();
      const uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
      visit([&](uint32_t key, uint32_t) {
        if ((key & pmask) == known) atomicAdd(&hist[(key >> lo) & (nb - 1u)], 1u);
      });
      __syncthreads();
      // largest digit d with count(digit >= d) >= need
      constexpr int PER = 2048 / kSelThreads;
      const int rb = kSelThreads - 1 - tid;           // reversed thread order
      uint32_t loc = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) loc += hist[rb * PER + i];
      uint32_t tot;
      const uint32_t above = block_excl_scan<kSelThreads>(loc, sh.scan, &tot);
      uint32_t run_c = above;
#pragma unroll
      for (int i = PER - 1; i >= 0; --i) {
        const uint32_t h = hist[rb * PER + i];
        if (run_c < need && run_c + h >= need) {
          misc[0] = (uint32_t)(rb * PER + i);
          misc[1] = run_c;
        }
        run_c += h;
      }
      __syncthreads();
      const uint32_t d = misc[0];
      need -= misc[1];
      known |= d << lo;
      hi = lo;
      __syncthreads();
    }
    kstar = known;
    take_eq = need;
  }
  // compaction in position order: keys above kstar, then the first take_eq equal to it
  uint32_t my_eq = 0;
  visit([&](uint32_t key, uint32_t) { my_eq += (key == kstar); });
  uint32_t tot;
  const uint32_t eq_base = block_excl_scan<kSelThreads>(my_eq, sh.scan, &tot);
  uint32_t my_sel = 0;
  {
    uint32_t er = eq_base;
    visit([&](uint32_t key, uint32_t) {
      if (key > kstar) ++my_sel;
      else if (key == kstar) { if (er < take_eq) ++my_sel; ++er; }
    });
  }
  const uint32_t sel_base = block_excl_scan<kSelThreads>(my_sel, sh.scan, &tot);
  int32_t* out = p.idx + (size_t)t * p.k;
  {
    uint32_t er = eq_base, o = sel_base;
    visit([&](uint32_t key, uint32_t pos) {
      bool s = false;
      if (key > kstar) s = true;
      else if (key == kstar) { s = er < take_eq; ++er; }
      if (s) {
        if (o < kk) out[o] = (int32_t)pos;
        ++o;
      }
    });
  }
  for (int i = (int)kk + tid; i < p.k; i += kSelThreads) out[i] = -1;
  if (tid == 0) {
    if (p.count) p.count[t] = (int32_t)kk;
    ast(p.ctl + ctl::kTau + t, 0u);
    ast(p.ctl + ctl::kDone + 64 * t, 0u);
  }
  __syncthreads();
}

template <int SRC, int KDT, int RT>
__global__ void __launch_bounds__(kSelThreads, 1) select_kernel(SelParams p) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int wg = blockIdx.x;
  const int64_t c0 = (int64_t)wg * p.chunk;
  const int T = p.T;
  // ---------------- P1: scores of this chunk into LDS, group maxima
  int64_t nkeys = p.L - c0;
  nkeys = nkeys < 0 ? 0 : (nkeys > p.chunk ? p.chunk : nkeys);
  if constexpr (SRC == 0) {
    Frag8 qa[RT][4];
    float wv[RT][16];
    load_q_frags<RT>(p.q_idx, T, qa);
    load_w<RT>(p.w_idx, T, wv);
    uint32_t gm[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) gm[r] = 0u;
    const int ntiles = (int)((nkeys + kTile - 1) / kTile);
    KeyTile<KDT> cur, nxt;
    int tile = wave;
    if (tile < ntiles) load_key_tile<KDT>(p.k_idx, p.k_scale, p.L, c0 + (int64_t)tile * kTile, cur);
    for (; tile < ntiles; tile += kSelWaves) {
      const int tn = tile + kSelWaves;
      if (tn < ntiles) load_key_tile<KDT>(p.k_idx, p.k_scale, p.L, c0 + (int64_t)tn * kTile, nxt);
      float out[RT];
      score_tile<KDT, RT>(cur, qa, wv, out);
      const int sl = tile * kTile + (lane & 31);
      const int64_t s = c0 + sl;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int tt = 2 * r + half;
        if (tt < T) {
          sh.sc[tt][sl] = out[r];
          if (s < p.L && s <= p.pos0 + tt) gm[r] = max(gm[r], order_key(out[r]));
        }
      }
      cur = nxt;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int tt = 2 * r + half;
      if (tt < T) sh.gmax[tt][wave * 32 + (lane & 31)] = gm[r];
    }
  } else {
    // scores from memory: coalesced reads, group g = elements g, g + kGroups, ...
    for (int t = 0; t < T; ++t) {
      const float* src = p.scores + (size_t)t * p.ld + c0;
      for (int i = tid; i < nkeys; i += kSelThreads) sh.sc[t][i] = src[i];
    }
    __syncthreads();
    for (int t = 0; t < T; ++t) {
      if (tid < kGroups) {
        uint32_t g = 0u;
        for (int i = tid; i < nkeys; i += kGroups) {
          const int64_t s = c0 + i;
          if (s <= p.pos0 + t) g = max(g, order_key(sh.sc[t][i]));
        }
        sh.gmax[t][tid] = g;
      }
    }
  }
  __syncthreads();
  // tau of this workgroup (one wave per token)
  if (p.m > 0 && wg < p.n_part) {
    for (int t = wave; t < T; t += kSelWaves) {
      const uint32_t tw = mth_largest_wave(sh.gmax[t], p.m);
      if (lane == 0) amax(p.ctl + ctl::kTau + t, ~tw);
    }
  }
  grid_barrier(p.ctl, p.nwg);
  // ---------------- P2: candidates >= tau in position order; the last workgroup to
  // publish a token's candidates resolves that token
  if (tid < T) {
    sh.tau[tid] = (p.m > 0) ? ~ald(p.ctl + ctl::kTau + tid) : 0u;
    sh.resolve[tid] = 0u;
  }
  __syncthreads();
  {
    const int per = (p.chunk + kSelThreads - 1) / kSelThreads;
    const int i0 = tid * per;
    for (int tt = 0; tt < T; ++tt) {
      const int t = (tt + wg) % T;            // rotate so different workgroups finish different tokens last
      const uint32_t tau = sh.tau[t];
      const int64_t lim = p.pos0 + t - c0;    // visible local indices: i <= lim and i < nkeys
      uint32_t c = 0;
      for (int i = i0; i < i0 + per; ++i)
        if (i < nkeys && i <= lim && order_key(sh.sc[t][i]) >= tau) ++c;
      uint32_t tot;
      uint32_t o = block_excl_scan<kSelThreads>(c, sh.scan, &tot);
      uint64_t* dst = p.cand + ((size_t)t * p.nwg + wg) * p.chunk;
      for (int i = i0; i < i0 + per; ++i) {
        if (i < nkeys && i <= lim) {
          const uint32_t key = order_key(sh.sc[t][i]);
          if (key >= tau) ast64(dst + o++, ((uint64_t)(uint32_t)(c0 + i) << 32) | key);
        }
      }
      if (tid == 0) ast(p.cnt + (size_t)t * p.nwg + wg, tot);
      vm_wait_all();
      __syncthreads();
      if (tid == 0) {
        if (aadd(p.ctl + ctl::kDone + 64 * t, 1u) == (uint32_t)p.nwg - 1u) sh.resolve[t] = 1u;
      }
    }
  }
  __syncthreads();
  // ---------------- P3: exact selection of the tokens this workgroup completed
  for (int t = 0; t < T; ++t)
    if (sh.resolve[t]) resolve_token(p, t, sh);
}

// ----------------------------------------------------------------------------- host launchers

static int row_tiles(int T) { return (T + 1) / 2; }

hipError_t launch_indexer_scores(const void* q_idx, const float* w_idx, const void* k_idx,
                                 const float* k_scale, int kdt, int T, int64_t L, int64_t pos0,
                                 float* scores, int64_t ld, hipStream_t st) {
  const int64_t ntiles = (L + kTile - 1) / kTile;
  const int64_t per_block = (kScoreThreads / 64) * kScoreTilesPerWave;
  const dim3 grid((unsigned)((ntiles + per_block - 1) / per_block));
  const dim3 block(kScoreThreads);
  const auto* q = static_cast<const uint16_t*>(q_idx);
  const auto* kk = static_cast<const uint8_t*>(k_idx);
#define DSA_SCORES(KD, RTv) \
  hipLaunchKernelGGL((indexer_scores_kernel<KD, RTv>), grid, block, 0, st, q, w_idx, kk, k_scale, T, L, pos0, scores, ld)
  const int rt = row_tiles(T);
  if (kdt == 0) {
    if (rt == 1) DSA_SCORES(0, 1); else if (rt == 2) DSA_SCORES(0, 2); else if (rt == 3) DSA_SCORES(0, 3); else DSA_SCORES(0, 4);
  } else {
    if (rt == 1) DSA_SCORES(1, 1); else if (rt == 2) DSA_SCORES(1, 2); else if (rt == 3) DSA_SCORES(1, 3); else DSA_SCORES(1, 4);
  }
#undef DSA_SCORES
  return hipGetLastError();
}

SelGeometry select_geometry(int T, int64_t L, int64_t pos0, int k, int num_cu) {
  SelGeometry g{};
  int64_t per = (L + num_cu - 1) / num_cu;
  int64_t chunk = ((per + 127) / 128) * 128;
  if (chunk < 128) chunk = 128;
  g.chunk = (int)chunk;
  int64_t nwg = (L + chunk - 1) / chunk;
  if (nwg < T) nwg = T;
  g.nwg = (int)nwg;
  g.fits = chunk <= kMaxChunk && nwg <= 1024;
  g.n_part = (int)(pos0 / chunk);
  const int64_t kmax = (int64_t)k < L ? k : L;
  g.m = 0;
  if (g.n_part >= 1) {
    const int64_t m = (kmax + g.n_part - 1) / g.n_part;
    if (m >= 1 && m <= kTauMaxM) g.m = (int)m;
  }
  return g;
}

size_t select_workspace_bytes(int T, int64_t L, int k, int num_cu) {
  SelGeometry g = select_geometry(T, L, L - T, k, num_cu);
  return ctl::kBytes + (size_t)kMaxT * 1024 * 4 + (size_t)kMaxT * g.nwg * g.chunk * sizeof(uint64_t);
}

int64_t select_max_context(int num_cu) { return (int64_t)num_cu * kMaxChunk; }

hipError_t launch_select(int src, const void* q_idx, const float* w_idx, const void* k_idx,
                         const float* k_scale, int kdt, const float* scores, int64_t ld, int T,
                         int64_t L, int64_t pos0, int k, int32_t* idx, int32_t* count, void* ws,
                         int num_cu, hipStream_t st) {
  SelGeometry g = select_geometry(T, L, pos0, k, num_cu);
  SelParams p{};
  p.q_idx = static_cast<const uint16_t*>(q_idx);
  p.w_idx = w_idx;
  p.k_idx = static_cast<const uint8_t*>(k_idx);
  p.k_scale = k_scale;
  p.scores = scores;
  p.ld = ld;
  p.T = T;
  p.k = k;
  p.L = L;
  p.pos0 = pos0;
  p.chunk = g.chunk;
  p.nwg = g.nwg;
  p.m = g.m;
  p.n_part = g.n_part;
  p.idx = idx;
  p.count = count;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  p.ctl = reinterpret_cast<uint32_t*>(w8);
  p.cnt = reinterpret_cast<uint32_t*>(w8 + ctl::kBytes);
  p.cand = reinterpret_cast<uint64_t*>(w8 + ctl::kBytes + (size_t)kMaxT * 1024 * 4);
  void* args[] = {&p};
  const int rt = row_tiles(T);
  void* fn = nullptr;
  if (src == 1) {
    fn = (void*)select_kernel<1, 0, 1>;
  } else if (kdt == 0) {
    fn = rt == 1 ? (void*)select_kernel<0, 0, 1> : rt == 2 ? (void*)select_kernel<0, 0, 2>
       : rt == 3 ? (void*)select_kernel<0, 0, 3> : (void*)select_kernel<0, 0, 4>;
  } else {
    fn = rt == 1 ? (void*)select_kernel<0, 1, 1> : rt == 2 ? (void*)select_kernel<0, 1, 2>
       : rt == 3 ? (void*)select_kernel<0, 1, 3> : (void*)select_kernel<0, 1, 4>;
  }
  // every workgroup must be resident at once (one per CU by the LDS footprint)
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kSelThreads, 0);
  if (e != hipSuccess) return e;
  if ((int64_t)per_cu * num_cu < g.nwg) return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel(fn, dim3(g.nwg), dim3(kSelThreads), args, 0, st);
}

}  // namespace dsa
