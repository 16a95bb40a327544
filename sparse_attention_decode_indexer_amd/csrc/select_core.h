// Device code of the indexer scan and the exact top-k selection, shared by the
// selection kernels and the fused DSA layer kernel.
//
// Method: NaiveAI research page on Naive-N0.5-Flash (naive.ai/en/research),
// §Model Architecture
// (the indexer scores the full history, the backbone attends a selected subset) and
// §Hybrid SWA-DSA Architecture (16 indexer heads, top 2,048 positions).
//
// Score of key s for token t:  I[t,s] = sum_h w[t,h] * relu(q_I[t,h] . k[s]) (* row scale).
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16): one row tile = 2 tokens x 16 heads = 32 MFMA
// rows; the 32 MFMA columns are 32 consecutive keys; K = 64 indexer dims in 4 steps.
// A block of 8 tokens therefore fills 128 rows with no padding.  The epilogue does
// relu -> x w -> fixed-order head sum in registers (each lane holds the 16 heads of one
// token) and, for e4m3 keys, one multiply by the row scale.
//
// Selection is one launch of one workgroup per chunk of C keys, all resident at once:
//   P1  scores of the chunk (computed, or read from memory) stay in LDS; each
//       workgroup derives a lower bound tau_wg of its m-th largest visible score from
//       per-group maxima and publishes it in its own slot;
//   --  tau = min over the slots (waiting until each carries this launch's tag);
//   P2  every workgroup writes its visible scores >= tau, in position order, as
//       (order key, position) candidates, then its count tagged with the launch;
//   P3  workgroup t waits until every count of token t carries this launch's tag,
//       runs an exact radix select over token t's candidates and writes the selected
//       positions in ascending order.
// There is no grid barrier: inter-workgroup data moves only through agent-scope atomic
// loads/stores of tagged slots, so no cache writeback or invalidation is needed.
// Because at least m scores of each of n_part workgroups are >= tau and
// m * n_part >= k, the candidates always contain the k best; the result is exact and
// independent of tau.  All cross-workgroup arithmetic is integer, so the result is
// bitwise reproducible.
#pragma once
#include <type_traits>

#include "dsa_common.h"
#include "select_geometry.h"

namespace dsa {

constexpr int kTile = 32;          // keys per MFMA column tile
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kPrefetch = 2;       // key tiles in flight per wave

// ----------------------------------------------------------------------------- tile math

template <int KDT>
struct KeyTile {
  uint4 raw[KDT == 0 ? 4 : 2];   // this lane's 32 dims of its key (bf16: 64 B, e4m3: 32 B)
  float scale;
};

// Lane l loads dims [32*(l>>5), +32) of key s0 + (l & 31); rows past L are clamped
// (their scores are never used).
template <int KDT, bool WITH_SCALE = true>
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
    if constexpr (WITH_SCALE) kt.scale = kscale[s];
  }
}

// Row scale of this lane's key in the tile at s0 (clamped like the keys)
DSA_DEV float load_key_scale(const float* __restrict__ kscale, int64_t L, int64_t s0) {
  int64_t s = s0 + (threadIdx.x & 31);
  s = s < L ? s : L - 1;
  return kscale[s];
}

// Rows of a score tile (2 tokens x 16 heads): row m holds token 2r + ((m >> 2) & 1) and
// head (m & 3) + 4 p(m >> 3) with p = (0, 2, 1, 3).  A lane of half c then receives, as
// its 16 accumulator elements (rows 8 (e >> 2) + 4 c + (e & 3)), all 16 heads of token
// 2r + c: elements 0-7 heads 0-3 and 8-11, elements 8-15 heads 4-7 and 12-15.
DSA_DEV int tile_row_token(int m) { return (m >> 2) & 1; }
DSA_DEV int tile_row_head(int m) { return (m & 3) + 4 * (((m >> 3) & 1) * 2 + (m >> 4)); }

// A operands of row tiles rt0 .. rt0+RTW-1, k-step j.  Lane l: row (l & 31) -> token
// 2r + tile_row_token(l & 31), head tile_row_head(l & 31); dims 32*(l>>5) + 8j .. +8 (the
// key operand's dims).
template <int RTW>
DSA_DEV void load_q_frags(const uint16_t* __restrict__ q_idx, int T, int rt0, Frag8 (&qa)[RTW][4]) {
  const int l = threadIdx.x & 63;
  const int half = l >> 5;
  const int row = l & 31;
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
    const int tt = 2 * (rt0 + r) + tile_row_token(row);
    const int tc = tt < T ? tt : T - 1;          // clamped: loads stay unconditional
    const int hh = tile_row_head(row);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qa[r][j].u = *reinterpret_cast<const uint4*>(q_idx + (tc * kHI + hh) * kDI + half * 32 + 8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tt >= T) qa[r][j].u = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Head weights of this lane's accumulator elements.  Element e of the 32x32 output holds
// row m = 8*(e>>2) + 4*half + (e&3): token 2r + half, head tile_row_head(m).
template <int RTW>
DSA_DEV void load_w(const float* __restrict__ w_idx, int T, int rt0, float (&wv)[RTW][16]) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tt = 2 * (rt0 + r) + half;
      const int hh = tile_row_head(8 * (e >> 2) + 4 * half + (e & 3));
      const float v = w_idx[(tt < T ? tt : T - 1) * kHI + hh];
      wv[r][e] = (tt < T) ? v : 0.0f;
    }
  }
}

// Staged query rows are padded from 64 to 72 bf16 (144 bytes): the fragment loads of 16
// heads at one column then fall in distinct banks instead of four.
constexpr int kQsRow = kDI + 8;

// Query block staged in LDS: qs [kMaxT][kHI][kQsRow] bf16 and wsh [kMaxT][kHI] fp32, rows of
// tokens >= T zero.  The loaders below read it with the same lane mapping and produce
// the same values as load_q_frags / load_w.
template <int RTW>
DSA_DEV void load_q_frags_lds(const uint16_t* qs, Frag8 (&qa)[RTW][4]) {
  static_assert(kQsRow % 8 == 0, "16-byte aligned rows");
  const int l = threadIdx.x & 63;
  const int half = l >> 5;
  const int row = l & 31;
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
    const int tt = 2 * r + tile_row_token(row);
    const int hh = tile_row_head(row);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qa[r][j].u = *reinterpret_cast<const uint4*>(qs + (tt * kHI + hh) * kQsRow + half * 32 + 8 * j);
  }
}

template <int RTW>
DSA_DEV void load_w_lds(const float* wsh, float (&wv)[RTW][16]) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {              // elements 4g .. 4g+3: four consecutive heads
      const int tt = 2 * r + half;
      const int hh = tile_row_head(8 * g);
      const float4 v = *reinterpret_cast<const float4*>(wsh + tt * kHI + hh);
      wv[r][4 * g + 0] = v.x;
      wv[r][4 * g + 1] = v.y;
      wv[r][4 * g + 2] = v.z;
      wv[r][4 * g + 3] = v.w;
    }
  }
}

// Order key without the -0 canonicalisation (3 instructions).  Only used where -0 may
// rank below +0 harmlessly (the tau lower bound).
DSA_DEV uint32_t order_key_fast(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Inverse of order_key on canonical keys: the float with that key (key 0 -> -inf side
// handled by the caller).
DSA_DEV float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// relu by integer max on the bit pattern: non-negative floats (sign 0) are non-negative
// integers, negative floats (and -0) are negative integers, so max(bits, 0) is relu(x)
// without a NaN canonicalisation.
DSA_DEV float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Building blocks of a tile's scores.  Their arithmetic and its order are fixed and the
// same in every kernel that uses them: per head a = q_h . k (MFMA, fp32); per lane, for
// its token, sum_e w_e relu(a_e) over heads 0-3, 8-11 and over heads 4-7, 12-15, each in
// element order, then the two added; then x the row scale for e4m3 keys.

// e4m3 or bf16 key tile -> the four bf16 B operands (e4m3 -> bf16 is exact)
template <int KDT>
DSA_DEV void keys_to_bf16(const KeyTile<KDT>& kt, Frag8 (&kb)[4]) {
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
}

// one 32-row tile against the key tile: K = 64 in four steps
DSA_DEV f32x16_t mma_k64(const Frag8 (&a)[4], const Frag8 (&kb)[4]) {
  f32x16_t acc = {};
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j].v, kb[j].v, acc, 0, 0, 0);
  return acc;
}

// score of token 2r + (lane>>5) for key lane & 31 from the row tile's accumulator
template <int KDT>
DSA_DEV float row_score(const f32x16_t& acc, const float (&w)[16], float scale) {
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) p0 = fmaf(w[e], relu_bits(acc[e]), p0);
#pragma unroll
  for (int e = 8; e < 16; ++e) p1 = fmaf(w[e], relu_bits(acc[e]), p1);
  // the lane holds all 16 heads of one token (the tile's row order): heads 0-3, 8-11 in
  // p0, heads 4-7, 12-15 in p1
  const float v = p0 + p1;
  return (KDT == 1) ? v * scale : v;
}

// Scores of one 32-key tile for RTW row tiles: out[r] is the score of token
// 2(rt0+r) + (lane>>5) for key s0 + (lane & 31).
template <int KDT, int RTW>
DSA_DEV void score_tile(const KeyTile<KDT>& kt, const Frag8 (&qa)[RTW][4], const float (&wv)[RTW][16],
                        float (&out)[RTW]) {
  Frag8 kb[4];
  keys_to_bf16<KDT>(kt, kb);
  out[0] = row_score<KDT>(mma_k64(qa[0], kb), wv[0], kt.scale);
  if constexpr (RTW > 1) out[1] = row_score<KDT>(mma_k64(qa[1], kb), wv[1], kt.scale);
  if constexpr (RTW > 2) out[2] = row_score<KDT>(mma_k64(qa[2], kb), wv[2], kt.scale);
  if constexpr (RTW > 3) out[3] = row_score<KDT>(mma_k64(qa[3], kb), wv[3], kt.scale);
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
  int chunk;             // keys per workgroup (multiple of 512, <= kMaxSpillChunk)
  int nwg;               // workgroups (>= T)
  int m;                 // tau rank; 0 disables tau
  int n_part;            // workgroups [0, n_part) publish tau
  // outputs
  int32_t* idx;
  int32_t* count;
  // workspace
  uint32_t* ctl;         // control words (see namespace ctl)
  uint64_t* cnt;         // [T][nwg] (launch tag << 32 | candidate count)
  uint64_t* tauv;        // [T][kMaxWG] (launch tag << 32 | tau bound) per workgroup
  uint64_t* cand;        // [T][nwg][chunk] (position << 32 | order key)
  uint64_t* trace;       // profiling builds: [nwg][16] phase timestamps
  float* spill;          // fused scan with chunk > kMaxChunk: scores of local positions
                         // >= kMaxChunk, [kMaxT][nwg][chunk - kMaxChunk]
  int64_t sstride;       // floats between the spill rows of consecutive tokens
};

struct SelShared {
  alignas(16) float sc[kMaxT][kMaxChunk];   // chunk scores (P1/P2); resolver scratch (P3); 16-byte reads
  float kscale[kMaxChunk];           // row scales of the chunk (e4m3 keys)
  uint32_t wcnt[2 * kSelWaves];      // resolver: per-wave counts
  float dump[64];                    // target of scores that are not kept (clamped tiles)
  uint32_t scan[32];
};

// m-th largest of the 64 values held by the lanes of one wave (1 <= m <= 64): the
// largest x with at least m lanes holding a value >= x, built bit by bit from the top
// (one compare and one ballot count per bit).
DSA_DEV uint32_t mth_largest_lanes(uint32_t v, int m) {
  uint32_t r = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = r | (1u << b);
    if (__builtin_popcountll(__ballot(v >= c)) >= m) r = c;
  }
  return r;
}

// A lower bound of the m-th largest that searches only the top NB bits (the rest zero):
// the largest x with its low 32 - NB bits clear and at least m lanes holding a value
// >= x.  It is at most the exact value and within one unit of bit 32 - NB of it.
template <int NB>
DSA_DEV uint32_t mth_largest_lanes_top(uint32_t v, int m) {
  uint32_t r = 0u;
#pragma unroll
  for (int b = 31; b >= 32 - NB; --b) {
    const uint32_t c = r | (1u << b);
    if (__builtin_popcountll(__ballot(v >= c)) >= m) r = c;
  }
  return r;
}

// The same when every lane that counts holds a value whose bits from `hi` up equal
// those of `known` (lower bits of `known` zero) and the other lanes hold 0, which no
// candidate key equals: only the low `hi` bits are searched.
DSA_DEV uint32_t mth_largest_lanes_below(uint32_t v, int m, uint32_t known, int hi) {
  uint32_t r = known;
  for (int b = hi - 1; b >= 0; --b) {
    const uint32_t c = r | (1u << b);
    if (__builtin_popcountll(__ballot(v >= c)) >= m) r = c;
  }
  return r;
}

// The tau bound keeps the top 16 bits of an order key (sign, exponent and 7 mantissa
// bits): lowering it by under 2^-7 relative admits a few percent more candidates and
// halves the bit search each workgroup runs before publishing its bound.
constexpr int kTauBits = 16;

constexpr int kRegPer = 16;                                  // candidates per lane
constexpr uint32_t kRegCands = kSelThreads * kRegPer;        // register-resident limit

// Boundary digit of a radix pass, by one wave: the largest digit d of the 4096-bin
// histogram with count(digit >= d) >= need (1 <= need <= the histogram's total).  Lane l
// sums bins [64 l, 64 l + 64) (reading its 16-byte chunks in a lane-rotated order, so the
// lanes of one read hit different banks); a scan over the lanes finds the lane range
// holding d, then one bin per lane of that range.  Writes d, the count of keys in digits
// above d and the count of digit d to misc[0..2], and clears misc[4] (the small-bin list
// counter).
DSA_DEV void radix_digit_wave(const uint32_t* hist, uint32_t need, uint32_t* misc) {
  const int lane = threadIdx.x & 63;
  const uint4* hp = reinterpret_cast<const uint4*>(hist + 64 * lane);
  uint32_t s = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 q = hp[(i + lane) & 15];
    s += (q.x + q.y) + (q.z + q.w);
  }
  const uint32_t inc = wave_incl_scan(s);
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63) - inc;   // bins of higher lanes
  // lanes whose range lies wholly below the boundary have `above` >= need; the first lane
  // with above < need holds d (the last lane always qualifies: above = 0)
  const int L = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(above < need)));
  const uint32_t sl = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
  const uint32_t h = hist[64 * L + lane];
  const uint32_t pre = wave_incl_scan(h);
  const uint32_t suf = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + h;          // bins >= this lane's
  // the largest digit of the range whose count from it upward reaches need
  const int dl = 63 - __builtin_clzll(__ballot(sl + suf >= need));
  if (lane == dl) {
    misc[0] = (uint32_t)(64 * L + dl);
    misc[1] = sl + suf - h;
    misc[2] = h;
    misc[4] = 0u;
  }
}

// Register-resident tail of the selection for nc <= kRegCands candidates already in LDS
// (position order): wave w holds elements [w*R, (w+1)*R) as NB 64-element blocks (lane
// = element), so ballots give position-ordered ranks.  Radix passes histogram the
// registers; the compaction counts per wave in one pass and writes in a second.
template <int NB>
DSA_DEV void resolve_regs(const SelParams& p, int t, SelShared& sh, const uint64_t* lc,
                          uint32_t nc, uint32_t kk, uint32_t kmin, uint32_t kmax,
                          uint32_t* hist, uint32_t* misc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t R = ((nc + kSelWaves - 1) / kSelWaves + 63) & ~63u;   // <= 64 * NB
  const uint32_t w0 = min(nc, (uint32_t)wave * R), w1 = min(nc, w0 + R);
  const uint32_t nmine = (w1 > w0 + lane) ? (w1 - w0 - lane + 63u) / 64u : 0u;
  uint64_t e[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint32_t g = w0 + 64u * i + lane;
    e[i] = lc[g < nc ? g : nc - 1];
  }
  block_minmax_u32<kSelThreads>(kmin, kmax, sh.scan);
  DSA_MARK(p.trace, 10);
  uint32_t kstar, take_eq;
  bool all_eq = false;                 // every key equal to the cut is taken (known early)
  if (kk == nc) {
    kstar = kmin;
    take_eq = 0xffffffffu;
    all_eq = true;
  } else {
    // MSB-first radix select on the bits where candidate keys differ: a first pass of 12
    // bits (4096 bins), then, when the boundary bin holds at most 64 keys, one wave
    // finds the cut among them directly; otherwise 11-bit passes continue
    const uint32_t diff = kmin ^ kmax;
    int hi = diff ? 32 - __builtin_clz(diff) : 0;
    uint32_t known = hi >= 32 ? 0u : (kmax & ~((1u << hi) - 1u));
    uint32_t need = kk;
    uint32_t* binl = hist + 4096;                                     // [64] keys of a small bin
    bool first = true;
    while (hi > 0) {
      const int maxd = first ? 12 : 11;
      const int dbits = hi < maxd ? hi : maxd;
      const int lo = hi - dbits;
      const uint32_t nb = 1u << dbits;
      if (!first) {                      // the first pass finds the histogram cleared
        for (int b2 = tid; b2 < 4096; b2 += kSelThreads) hist[b2] = 0u;
        __syncthreads();
      }
      first = false;
      const uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const uint32_t key = (uint32_t)e[i];
        if (((uint32_t)i < nmine) & ((key & pmask) == known)) atomicAdd(&hist[(key >> lo) & (nb - 1u)], 1u);
      }
      __syncthreads();
      // the boundary digit, found by wave 0 alone while the other waves wait at one barrier
      if (wave == 0) radix_digit_wave(hist, need, misc);
      __syncthreads();
      const uint32_t d = misc[0];
      need -= misc[1];
      known |= d << lo;
      hi = lo;
      const uint32_t in_bin = misc[2];
      if (hi == 0) all_eq = need == in_bin;   // the last digit fixed every bit
      if (need == in_bin && hi > 0) {
        // the whole boundary bin is taken: the cut is its smallest key
        const uint32_t pm = ~((1u << hi) - 1u);
        uint32_t bmin = 0xffffffffu;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const uint32_t key = (uint32_t)e[i];
          if (((uint32_t)i < nmine) & ((key & pm) == known)) bmin = min(bmin, key);
        }
        known = block_min_u32<kSelThreads>(bmin, sh.scan);
        need = 0xffffffffu;      // every key equal to the cut is taken
        all_eq = true;
        hi = 0;
      } else if (hi > 0 && in_bin <= 64u) {
        // small boundary bin: gather its keys (any order; misc[4] was cleared with the
        // digit) and let wave 0 take the need-th largest; `need` then counts the keys
        // equal to it that are taken
        const uint32_t pm = ~((1u << hi) - 1u);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const uint32_t key = (uint32_t)e[i];
          if (((uint32_t)i < nmine) & ((key & pm) == known)) binl[atomicAdd(&misc[4], 1u)] = key;
        }
        __syncthreads();
        if (wave == 0) {
          const bool mine = (uint32_t)lane < in_bin;
          const uint32_t v = mine ? binl[lane] : 0u;
          const uint32_t cut = mth_largest_lanes_below(v, (int)need, known, hi);
          const uint32_t gt = (uint32_t)__builtin_popcountll(__ballot(mine & (v > cut)));
          const uint32_t eq = (uint32_t)__builtin_popcountll(__ballot(mine & (v == cut)));
          if (lane == 0) {
            misc[0] = cut;
            misc[1] = need - gt;
            misc[3] = eq == need - gt;   // the bin holds every key equal to the cut
          }
        }
        __syncthreads();
        known = misc[0];
        need = misc[1];
        all_eq = misc[3] != 0u;
        hi = 0;                          // misc is not written again in this call
      }
    }
    kstar = known;
    take_eq = need;
  }
  DSA_MARK(p.trace, 11);
  // Compaction in position order: per-wave counts give each wave's first output slot.
  // When every key equal to the cut is taken (known from the radix step, or found from
  // the counts) a key is selected iff it is >= the cut and one count per wave suffices;
  // otherwise keys above and equal to the cut are counted apart and the first take_eq
  // equal keys in position order are taken.
  int32_t* out = p.idx + (size_t)t * p.k;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t* wq = sh.wcnt;           // [8] selected (or above) counts, then [8] equal counts
  uint32_t o = 0, er = 0;
  if (all_eq) {
    uint32_t cs = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      cs += (uint32_t)__builtin_popcountll(__ballot(((uint32_t)i < nmine) & ((uint32_t)e[i] >= kstar)));
    }
    if (lane == 0) wq[wave] = cs;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSelWaves; ++j) o += j < wave ? wq[j] : 0u;
  } else {
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t key = (uint32_t)e[i];
      const bool v = (uint32_t)i < nmine;
      cgt += (uint32_t)__builtin_popcountll(__ballot(v & (key > kstar)));
      ceq += (uint32_t)__builtin_popcountll(__ballot(v & (key == kstar)));
    }
    if (lane == 0) { wq[wave] = cgt; wq[kSelWaves + wave] = ceq; }
    __syncthreads();
    uint32_t eb = 0;
#pragma unroll
    for (int j = 0; j < kSelWaves; ++j) {
      const uint32_t gj = wq[j], ej = wq[kSelWaves + j];
      const uint32_t rem = take_eq > eb ? take_eq - eb : 0u;
      const uint32_t sj = gj + (ej < rem ? ej : rem);
      if (j < wave) { er += ej; o += sj; }
      eb += ej;
    }
    all_eq = eb <= take_eq;
  }
  if (all_eq) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bool sel = ((uint32_t)i < nmine) & ((uint32_t)e[i] >= kstar);
      const uint64_t ms = __ballot(sel);
      const uint32_t oo = o + (uint32_t)__builtin_popcountll(ms & lt);
      if (sel & (oo < kk)) out[oo] = (int32_t)(e[i] >> 32);
      o += (uint32_t)__builtin_popcountll(ms);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t key = (uint32_t)e[i];
      const bool v = (uint32_t)i < nmine;
      const bool eq = v & (key == kstar);
      const uint64_t me = __ballot(eq);
      const bool sel = v & ((key > kstar) | (eq & (er + (uint32_t)__builtin_popcountll(me & lt) < take_eq)));
      const uint64_t ms = __ballot(sel);
      const uint32_t oo = o + (uint32_t)__builtin_popcountll(ms & lt);
      if (sel & (oo < kk)) out[oo] = (int32_t)(e[i] >> 32);
      er += (uint32_t)__builtin_popcountll(me);
      o += (uint32_t)__builtin_popcountll(ms);
    }
  }
  DSA_MARK(p.trace, 12);
  for (int i = (int)kk + tid; i < p.k; i += kSelThreads) out[i] = -1;
  if (tid == 0 && p.trace) p.trace[blockIdx.x * 16 + 13] = nc;
  if (tid == 0 && p.count) p.count[t] = (int32_t)kk;
  __syncthreads();
}

// Selection for a launch of one workgroup that holds every score of its single token
// (row 0 of the chunk scores): every visible score is a candidate, in position order --
// the candidates, and so the selection, of the path over several workgroups -- built in
// LDS rows 4-5, with the radix histogram and scratch in rows 2-3, then the register
// select.
static_assert(2 * kMaxChunk * 4 >= (4096 + 64 + 16) * 4 && 2 * kMaxChunk * 4 >= kMaxChunk * 8, "single-workgroup LDS use");
DSA_DEV void resolve_local(const SelParams& p, SelShared& sh, int nkeys) {
  const int tid = threadIdx.x;
  uint32_t* hist = reinterpret_cast<uint32_t*>(&sh.sc[2][0]);          // [4096] + [64] bin list
  uint32_t* misc = hist + 4096 + 64;
  uint64_t* lc = reinterpret_cast<uint64_t*>(&sh.sc[4][0]);            // [nc] (position, key)
  const int64_t vis = p.pos0 + 1;
  const uint32_t nc = (uint32_t)(vis < nkeys ? vis : nkeys);
  const uint32_t kk = (uint32_t)p.k < nc ? (uint32_t)p.k : nc;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int b2 = tid; b2 < 4096; b2 += kSelThreads) hist[b2] = 0u;
  for (uint32_t g = tid; g < nc; g += kSelThreads) {
    const uint32_t key = order_key(sh.sc[0][g]);
    lc[g] = ((uint64_t)g << 32) | key;
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
  __syncthreads();
  resolve_regs<8>(p, 0, sh, lc, nc, kk, kmin, kmax, hist, misc);
}

// Exact selection of the kk best candidates of token t.  Runs in one workgroup after
// every workgroup has published its candidates (after the second grid barrier).
// Candidates arrive in position order; the selection is: every key above the cut key
// K*, then the first `take_eq` (in position order) of the keys equal to K*.
DSA_DEV void resolve_token(const SelParams& p, int t, SelShared& sh, uint32_t epoch) {
  uint32_t* pre = reinterpret_cast<uint32_t*>(&sh.sc[0][0]);         // [nwg + 1]
  uint32_t* hist = pre + 1040;                                        // [4096] + [64] bin list
  uint32_t* misc = hist + 4096 + 64;                                  // small
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwg = p.nwg;
  const uint64_t* cnt_t = p.cnt + (size_t)t * nwg;
  // Each workgroup publishes its count, tagged with this launch, after its candidates;
  // waiting for all tags replaces a grid barrier and delivers the counts at once.
  constexpr int kCntPer = kMaxWG / kSelThreads;
  const uint32_t tag = epoch + 1u;
  uint32_t cw[kCntPer];
  bool gave_up = false;
  {
    uint64_t v[kCntPer];
#pragma unroll
    for (int j = 0; j < kCntPer; ++j) {
      const int w = tid + j * kSelThreads;
      v[j] = ald64(cnt_t + (w < nwg ? w : nwg - 1));
    }
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
    for (int j = 0; j < kCntPer; ++j) {
      const int w = tid + j * kSelThreads;
      while ((uint32_t)(v[j] >> 32) != tag) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
          ast(p.ctl + ctl::kError, 1u);
          v[j] = 0;
          gave_up = true;
          break;
        }
        v[j] = ald64(cnt_t + (w < nwg ? w : nwg - 1));
      }
      cw[j] = (w < nwg) ? (uint32_t)v[j] : 0u;
    }
  }
  if (__syncthreads_or(gave_up)) {
    // not every workgroup published (they were not all resident): this token's selection
    // is empty, the error word is set, and the launch counter stays as it is -- a
    // workgroup that has not run yet reads it later and tags with this launch
    int32_t* out = p.idx + (size_t)t * p.k;
    for (int i = tid; i < p.k; i += kSelThreads) out[i] = -1;
    if (tid == 0 && p.count) p.count[t] = 0;
    return;
  }
  DSA_MARK(p.trace, 8);
  // every workgroup has published, so every workgroup has read the launch counter
  if (t == 0 && tid == 0) ast(p.ctl + ctl::kEpoch, next_epoch(epoch));
  // prefix over workgroup counts
  uint32_t carry = 0;
#pragma unroll
  for (int j = 0; j < kCntPer; ++j) {
    const int base = j * kSelThreads;
    if (base >= nwg) break;
    const int w = base + tid;
    const uint32_t c = cw[j];
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
  // Bring the candidates on chip when they fit.  Wave w copies source segments w, w+8,
  // ...; one load instruction covers two of them (lanes 0-31 and 32-63, element = lane &
  // 31), since most segments hold fewer than 32 candidates.  Elements 32-63 follow in a
  // second batch when one of the wave's segments is that long, longer runs in a loop.
  uint64_t* lc = reinterpret_cast<uint64_t*>(misc + 16);              // 8-byte aligned
  const uint32_t lds_cap = (uint32_t)((sizeof(sh.sc) - (1040 + 4096 + 64 + 16) * 4) / 8);
  const bool in_lds = nc > 0 && nc <= lds_cap;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if (in_lds) {
    // the first radix pass finds its histogram cleared (separate from pre[] and lc[])
    for (int b2 = tid; b2 < 4096; b2 += kSelThreads) hist[b2] = 0u;
    constexpr int UP = 16;                                            // segment pairs per round
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int hl = lane >> 5;
    const uint32_t el = (uint32_t)lane & 31u;
    for (int s0 = wv; s0 < nwg; s0 += kSelWaves * 2 * UP) {
      uint32_t b0[UP], n[UP], so[UP];
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        const int sg = s0 + kSelWaves * (2 * u + hl);
        const int sc = sg < nwg ? sg : nwg - 1;
        const uint32_t x0 = pre[sc], x1 = pre[sc + 1];
        b0[u] = x0;
        n[u] = sg < nwg ? x1 - x0 : 0u;
        so[u] = (uint32_t)sc * (uint32_t)p.chunk;                     // < kMaxWG * kMaxChunk
      }
      uint64_t v[UP];
      // slot 0 of every segment exists, so the clamped reads stay in the workspace
#pragma unroll
      for (int u = 0; u < UP; ++u) v[u] = ald64(base + so[u] + (el < n[u] ? el : 0u));
      bool lng = false;
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        if (el < n[u]) {
          lc[b0[u] + el] = v[u];
          kmin = min(kmin, (uint32_t)v[u]);
          kmax = max(kmax, (uint32_t)v[u]);
        }
        lng |= n[u] > 32u;
      }
      if (__ballot(lng) != 0ull) {
#pragma unroll
        for (int u = 0; u < UP; ++u) v[u] = ald64(base + so[u] + (el + 32u < n[u] ? el + 32u : 0u));
        bool vlong = false;
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          if (el + 32u < n[u]) {
            lc[b0[u] + 32u + el] = v[u];
            kmin = min(kmin, (uint32_t)v[u]);
            kmax = max(kmax, (uint32_t)v[u]);
          }
          vlong |= n[u] > 64u;
        }
        if (__ballot(vlong) != 0ull) {
          // longer runs (short contexts without a bound: every visible score of a chunk is
          // a candidate) in rounds of eight loads per lane issued before any is used, so a
          // 512-candidate run takes two round trips instead of fourteen
          constexpr int LB = 8;
#pragma unroll 1
          for (int u = 0; u < UP; ++u) {
            for (uint32_t j0 = 64u; j0 < n[u]; j0 += 32u * LB) {
              uint64_t x[LB];
#pragma unroll
              for (int i = 0; i < LB; ++i) {
                const uint32_t j = j0 + el + 32u * i;
                x[i] = ald64(base + so[u] + (j < n[u] ? j : 0u));
              }
#pragma unroll
              for (int i = 0; i < LB; ++i) {
                const uint32_t j = j0 + el + 32u * i;
                if (j < n[u]) {
                  lc[b0[u] + j] = x[i];
                  kmin = min(kmin, (uint32_t)x[i]);
                  kmax = max(kmax, (uint32_t)x[i]);
                }
              }
            }
          }
        }
      }
    }
    __syncthreads();
    DSA_MARK(p.trace, 9);
    if (nc <= kRegCands) {
      // blocks of 64 candidates per wave: the register passes are unrolled to that many
      const uint32_t nb = (((nc + kSelWaves - 1) / kSelWaves + 63) & ~63u) / 64u;
      if (nb <= 8u) resolve_regs<8>(p, t, sh, lc, nc, kk, kmin, kmax, hist, misc);
      else if (nb <= 12u) resolve_regs<12>(p, t, sh, lc, nc, kk, kmin, kmax, hist, misc);
      else resolve_regs<kRegPer>(p, t, sh, lc, nc, kk, kmin, kmax, hist, misc);
      return;
    }
  }
  // element g of the position-ordered candidate list (LDS, or the workspace slots)
  auto elem = [&](uint32_t g) -> uint64_t {
    if (in_lds) return lc[g];
    int lo = 0, hi = nwg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return ald64(base + (size_t)lo * p.chunk + (g - pre[lo]));
  };
  // order-free passes read element g = tid, tid + 512, ... (conflict-free in LDS)
  if (!in_lds) {
    for (uint32_t g = tid; g < nc; g += kSelThreads) {
      const uint32_t key = (uint32_t)elem(g);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  }
  block_minmax_u32<kSelThreads>(kmin, kmax, sh.scan);
  DSA_MARK(p.trace, 10);
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
      for (int b2 = tid; b2 < 2048; b2 += kSelThreads) hist[b2] = 0u;
      __syncthreads();
      const uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
      for (uint32_t g0 = tid; g0 < nc; g0 += 4 * kSelThreads) {
        uint32_t key[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t g = g0 + u * kSelThreads;
          key[u] = (uint32_t)elem(g < nc ? g : nc - 1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if ((g0 + u * kSelThreads < nc) & ((key[u] & pmask) == known))
            atomicAdd(&hist[(key[u] >> lo) & (nb - 1u)], 1u);
      }
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
      const uint32_t in_bin = hist[d];
      __syncthreads();
      if (need == in_bin && hi > 0) {
        // the whole boundary bin is taken: the cut is its smallest key
        const uint32_t pm = ~((1u << hi) - 1u);
        uint32_t bmin = 0xffffffffu;
        for (uint32_t g = tid; g < nc; g += kSelThreads) {
          const uint32_t key = (uint32_t)elem(g);
          if ((key & pm) == known) bmin = min(bmin, key);
        }
        known = block_min_u32<kSelThreads>(bmin, sh.scan);
        need = 0xffffffffu;      // every key equal to the cut is taken
        hi = 0;
      }
    }
    kstar = known;
    take_eq = need;
  }
  DSA_MARK(p.trace, 11);
  // Position-ordered compaction: wave w owns elements [w*R, (w+1)*R) in 64-element
  // segments (lane = element), so ballots give in-order ranks.  Pass 1 counts keys equal
  // to K* per wave; pass 2 (knowing each wave's first equal-key rank) counts selected
  // elements; pass 3 writes.
  const uint32_t R = ((nc + kSelWaves - 1) / kSelWaves + 63) & ~63u;
  const uint32_t w0 = min(nc, wave * R), w1 = min(nc, w0 + R);
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t* wq = sh.wcnt;           // [8] equal counts, then [8] selected counts
  uint32_t cnt_eq = 0;
  for (uint32_t g0 = w0; g0 < w1; g0 += 64) {
    const uint32_t g = g0 + lane;
    const uint32_t key = (uint32_t)elem(g < w1 ? g : w1 - 1);
    const bool e = (g < w1) & (key == kstar);
    cnt_eq += (uint32_t)__builtin_popcountll(__ballot(e));
  }
  if (lane == 0) wq[wave] = cnt_eq;
  __syncthreads();
  uint32_t eq_base = 0;
  for (int j = 0; j < wave; ++j) eq_base += wq[j];
  uint32_t cnt_sel = 0;
  {
    uint32_t er = eq_base;
    for (uint32_t g0 = w0; g0 < w1; g0 += 64) {
      const uint32_t g = g0 + lane;
      const uint32_t key = (uint32_t)elem(g < w1 ? g : w1 - 1);
      const bool in = g < w1;
      const bool e = in & (key == kstar);
      const uint64_t me = __ballot(e);
      const bool sel = in & ((key > kstar) | (e & (er + (uint32_t)__builtin_popcountll(me & lt) < take_eq)));
      cnt_sel += (uint32_t)__builtin_popcountll(__ballot(sel));
      er += (uint32_t)__builtin_popcountll(me);
    }
  }
  __syncthreads();
  if (lane == 0) wq[8 + wave] = cnt_sel;
  __syncthreads();
  uint32_t sel_base = 0;
  for (int j = 0; j < wave; ++j) sel_base += wq[8 + j];
  int32_t* out = p.idx + (size_t)t * p.k;
  {
    uint32_t er = eq_base, o = sel_base;
    for (uint32_t g0 = w0; g0 < w1; g0 += 64) {
      const uint32_t g = g0 + lane;
      const uint64_t ev = elem(g < w1 ? g : w1 - 1);
      const uint32_t key = (uint32_t)ev;
      const bool in = g < w1;
      const bool e = in & (key == kstar);
      const uint64_t me = __ballot(e);
      const bool sel = in & ((key > kstar) | (e & (er + (uint32_t)__builtin_popcountll(me & lt) < take_eq)));
      const uint64_t ms = __ballot(sel);
      const uint32_t oo = o + (uint32_t)__builtin_popcountll(ms & lt);
      if (sel && oo < kk) out[oo] = (int32_t)(ev >> 32);
      er += (uint32_t)__builtin_popcountll(me);
      o += (uint32_t)__builtin_popcountll(ms);
    }
  }
  DSA_MARK(p.trace, 12);
  for (int i = (int)kk + tid; i < p.k; i += kSelThreads) out[i] = -1;
  if (tid == 0 && p.trace) p.trace[blockIdx.x * 16 + 13] = nc;
  if (tid == 0 && p.count) p.count[t] = (int32_t)kk;
  __syncthreads();
}

// The selection of one launch (all phases; workgroup t < T resolves token t).  Returns
// false, having written empty selections, when the workspace's error word was already
// set; otherwise true, with this launch's counter in `epoch_out` (slot tag = epoch + 1).
// SPILL: chunks longer than kMaxChunk keys.  The first kMaxChunk scores of the chunk stay
// in LDS; the fused scan writes the rest to the workspace's spill rows and the pass that
// emits candidates reads them from there (loaded scores are read again from the input).
// Every step is the same, so the selection is the one the exact top-k defines.
template <int SRC, int KDT, int RTW, bool SINGLE = false, bool SPILL = false>
DSA_DEV bool select_body(const SelParams& p, SelShared& sh, uint32_t& epoch_out) {
  static_assert(!(SINGLE && SPILL), "one workgroup holds at most kMaxChunk keys");
  static_assert(RTW >= 1 && RTW <= 4, "a wave holds one to four row tiles");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int wg = blockIdx.x;
  const int64_t c0 = (int64_t)wg * p.chunk;
  const int T = p.T;
  DSA_MARK(p.trace, 0);
  // The launch counter and the error word (read with one device-scope load, slow to
  // return) are requested after the prologue's loads, so that waiting for the queries and
  // the first key tiles does not wait for them; they are first needed when the tau bound
  // is published.
  uint64_t ctlw = 0u;
  // ---------------- P1: scores of this chunk into LDS
  int64_t nk64 = p.L - c0;
  nk64 = nk64 < 0 ? 0 : (nk64 > p.chunk ? p.chunk : nk64);
  const int nkeys = (int)nk64;
  // running maximum of this lane's scores per row tile (the tau bound's group maxima)
  float gmax[RTW];
#pragma unroll
  for (int r = 0; r < RTW; ++r) gmax[r] = -__builtin_inff();
  if constexpr (SRC == 0) {
    // wave w takes key tiles w, w + 8, ... and scores them for every row tile
    // (bf16 key tiles take twice the registers: one in flight when four row tiles are held)
    constexpr int PF = (KDT == 0 && RTW >= 3) ? 1 : kPrefetch;
    const int ntiles = (nkeys + kTile - 1) / kTile;
    const int nmine = ntiles > wave ? (ntiles - wave + kSelWaves - 1) / kSelWaves : 0;
    const int jlast = nmine > 0 ? nmine - 1 : 0;
    // Loads are unconditional (tile index clamped to the wave's last tile, which is then
    // already cached; rows past L are clamped inside) so the compiler keeps PF
    // tiles in flight without draining the memory counter at branch merges.
    auto tile_of = [&](int j) { return c0 + (int64_t)(wave + (j < jlast ? j : jlast) * kSelWaves) * kTile; };
    // The block's queries and head weights are staged in LDS (the score area is free
    // until the scan starts); their loads go out first, then the first key tiles (with
    // their row scales), whose latency overlaps the query set-up below.
    uint16_t* qs = reinterpret_cast<uint16_t*>(&sh.sc[0][0]);        // [kMaxT][kHI][kQsRow]
    float* wsh = &sh.sc[2][0];                                        // [kMaxT][kHI]
    static_assert(kMaxT * kHI * kQsRow * 2 <= 2 * kMaxChunk * 4, "padded query block fits two score rows");
    constexpr int QROW = kHI * kDI / 8;                               // uint4 per token
    constexpr int QPER = kMaxT * QROW / kSelThreads;
    static_assert(kMaxT * QROW % kSelThreads == 0 && kMaxT * kHI / 4 <= kSelThreads, "staging split");
    uint4 qv[QPER];
#pragma unroll
    for (int u = 0; u < QPER; ++u) {
      const int i = tid + u * kSelThreads;
      const int tq = i / QROW;
      qv[u] = reinterpret_cast<const uint4*>(p.q_idx)[(tq < T ? tq : T - 1) * QROW + i % QROW];
    }
    float4 w4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int tw = tid >> 2;
    if (tid < kMaxT * kHI / 4) w4 = reinterpret_cast<const float4*>(p.w_idx)[(tw < T ? tw : T - 1) * 4 + (tid & 3)];
    KeyTile<KDT> buf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) load_key_tile<KDT, true>(p.k_idx, p.k_scale, p.L, tile_of(i), buf[i]);
#pragma unroll
    for (int u = 0; u < QPER; ++u) {
      const int i = tid + u * kSelThreads;
      const int row = i / (kDI / 8), c8 = i % (kDI / 8);                // (token, head) row, 8-element chunk
      *reinterpret_cast<uint4*>(qs + row * kQsRow + 8 * c8) = (i / QROW < T) ? qv[u] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid < kMaxT * kHI / 4)
      reinterpret_cast<float4*>(wsh)[tid] = tw < T ? w4 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
    Frag8 qa[RTW][4];
    float wv[RTW][16];
    load_q_frags_lds<RTW>(qs, qa);
    load_w_lds<RTW>(wsh, wv);
    __syncthreads();                     // the staged block is read; the scan overwrites it
    ctlw = ald64(reinterpret_cast<const uint64_t*>(p.ctl + ctl::kEpoch));
    DSA_MARK(p.trace, 1);
    DSA_MARK_CLK(p.trace, 14);
    if (nmine > 0) {
      // Row tile r's epilogue runs on the vector units while the matrix cores work on row
      // tile r + 1.  Scores of clamped repeats go to a dump slot (selected by address, so
      // no branch splits the schedule).
      for (int base = 0; base < nmine; base += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          const int j = base + i;
          const int jc = j < nmine ? j : nmine - 1;      // the tile actually loaded (clamped)
          const int sl = (wave + jc * kSelWaves) * kTile + (lane & 31);
          const float scale = buf[i].scale;
          const bool keep = j < nmine;
          Frag8 kb[4];
          keys_to_bf16<KDT>(buf[i], kb);
          load_key_tile<KDT, false>(p.k_idx, p.k_scale, p.L, tile_of(j + PF), buf[i]);
          f32x16_t acc = mma_k64(qa[0], kb);
          // SPILL: a tile lies wholly before or after local position kMaxChunk (a multiple
          // of the tile), so the choice of LDS or spill row is uniform over the wave
          const bool spill_tile = SPILL && keep && (wave + jc * kSelWaves) * kTile >= kMaxChunk;
          float* row = keep && !spill_tile ? &sh.sc[half][sl] : &sh.dump[lane];
          const int rstride = keep && !spill_tile ? 2 * kMaxChunk : 0;  // floats between row tiles' rows
          float* grow = nullptr;
          if constexpr (SPILL)
            grow = p.spill + (size_t)half * p.sstride + (size_t)wg * (p.chunk - kMaxChunk) + (sl - kMaxChunk);
#pragma unroll
          for (int r = 0; r < RTW; ++r) {
            f32x16_t nxt = {};
            if (r + 1 < RTW) nxt = mma_k64(qa[r + 1 < RTW ? r + 1 : r], kb);
            const float o = row_score<KDT>(acc, wv[r], scale);
            gmax[r] = fmaxf(gmax[r], o);
            if constexpr (SPILL) {
              if (spill_tile) grow[(size_t)r * 2 * p.sstride] = o;
              else row[r * rstride] = o;
            } else {
              row[r * rstride] = o;
            }
            acc = nxt;
          }
          // the next scale of this slot is requested once the current one is used up, so
          // the two never live at once (no copy at the loop's back edge, whose wait would
          // drain every load in flight)
          if constexpr (KDT == 1) buf[i].scale = load_key_scale(p.k_scale, p.L, tile_of(j + PF));
        }
        // Issue order of the block's tiles (four row tiles): every MFMA is followed by up to
        // ten vector instructions, so one row tile's epilogue issues under the next row
        // tile's matrix work.  Left to itself the compiler issues a tile's MFMAs back to back.
        if constexpr (RTW == 4) {
#pragma unroll
          for (int g = 0; g < 4 * RTW * PF; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // then up to ten vector ALU
          }
        }
      }
    }
  } else {
    ctlw = ald64(reinterpret_cast<const uint64_t*>(p.ctl + ctl::kEpoch));
    constexpr int PER = kMaxChunk / kSelThreads;
    // a workgroup past the last key (nwg = T > ceil(L / chunk)) reads no scores
    for (int t = 0; t < (nkeys > 0 ? T : 0); ++t) {
      const float* src = p.scores + (size_t)t * p.ld + c0;
      float v[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int i = tid + q * kSelThreads;
        v[q] = src[i < nkeys ? i : nkeys - 1];
      }
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int i = tid + q * kSelThreads;
        if (i < nkeys) sh.sc[t][i] = v[q];
      }
    }
  }
  const uint32_t epoch = (uint32_t)ctlw;
  const uint32_t tag = epoch + 1u;                       // this launch's slot tag
  if constexpr (SPILL) __threadfence_block();            // spilled scores seen by every wave
  __syncthreads();
  DSA_MARK(p.trace, 2);
  // A workspace whose error word is set (an earlier launch on it gave up waiting) is not
  // trusted: the launch publishes nothing and writes an empty selection, until the
  // workspace is cleared again.
  epoch_out = epoch;
  if ((ctlw >> 32) != 0u) {
    if (wg < T) {
      int32_t* out = p.idx + (size_t)wg * p.k;
      for (int i = tid; i < p.k; i += kSelThreads) out[i] = -1;
      if (tid == 0 && p.count) p.count[wg] = 0;
    }
    return false;
  }
  if (wg >= T) DSA_MARK_CLK(p.trace, 13);     // core clock over P1 (profiling builds)
  if constexpr (SINGLE) {
    // one token, the whole context in this workgroup: select on chip.  The launch counter
    // still advances once (the workgroup has read it), as every selection launch does.
    if (tid == 0) ast(p.ctl + ctl::kEpoch, next_epoch(epoch));
    resolve_local(p, sh, nkeys);
    return true;
  }
  // ---------------- tau bound.  Any split of the chunk's (visible) scores into at least
  // m non-empty groups gives one: the m-th largest group maximum is <= the m-th largest
  // score.  Computed scores use 64 groups per token: the keys at one position mod 32
  // in the tiles of one index parity; loaded scores use 64 groups of
  // stride 64.  Only workgroups whose chunk lies entirely before pos0 publish, so every
  // score of the chunk is visible to every token.
  if (p.m > 0 && wg < p.n_part) {
    if constexpr (SRC == 0) {
      // group (token, wave, key lane) maxima -> LDS (the row-scale area is free now);
      // wave t then merges, per lane, the waves of one parity: 64 groups of the token
      constexpr int GPT = kSelWaves * 32;                           // group maxima per token
      float* gm = sh.kscale;                                        // [kMaxT][GPT]
      // the thread's row and wave are formed again from an opaque copy of its index, so
      // no value derived from it stays live (in a spill slot) across the scan
      int tid_o = threadIdx.x;
      asm volatile("" : "+v"(tid_o));
      const int half_o = (tid_o >> 5) & 1, wave_o = tid_o >> 6;
#pragma unroll
      for (int r = 0; r < RTW; ++r) {
        const int tt = 2 * r + half_o;
        if (tt < T) gm[tt * GPT + wave_o * 32 + (tid_o & 31)] = gmax[r];
      }
      __syncthreads();
      for (int t = wave; t < T; t += kSelWaves) {
        uint32_t g = 0u;
#pragma unroll
        for (int i = 0; i < GPT / 64; ++i) g = max(g, order_key_fast(gm[t * GPT + 64 * i + lane]));
        const uint32_t tw = mth_largest_lanes_top<kTauBits>(g, p.m);
        if (lane == 0) ast64(p.tauv + (size_t)t * kMaxWG + wg, ((uint64_t)tag << 32) | tw);
      }
    } else {
      for (int t = wave; t < T; t += kSelWaves) {
        uint32_t g = 0u;
        // (a longer chunk's bound comes from its first kMaxChunk scores: any subset of
        // the chunk's scores gives a valid one)
        const int nkt = SPILL && nkeys > kMaxChunk ? kMaxChunk : nkeys;
        for (int i0 = 0; i0 < nkt; i0 += 512) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = sh.sc[t][(i0 + u * 64 + lane) & (kMaxChunk - 1)];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (i0 + u * 64 + lane < nkt) g = max(g, order_key_fast(v[u]));
        }
        const uint32_t tw = mth_largest_lanes_top<kTauBits>(g, p.m);
        if (lane == 0) ast64(p.tauv + (size_t)t * kMaxWG + wg, ((uint64_t)tag << 32) | tw);
      }
    }
  }
  DSA_MARK(p.trace, 3);
  // ---------------- P2: wave t takes token t: tau = min of the published bounds, then
  // the chunk's visible scores >= tau go out in position order (one ballot per 64
  // positions, running offset) and the wave publishes their count.  Workgroup t alone
  // gathers token t's bounds and republishes their minimum in one tagged slot, which
  // every other workgroup polls (a single address instead of n_part slots per poller).
  if (wave < T) {
    const int t = wave;
    uint32_t tm = 0u;
    if (p.m > 0) {
      uint64_t* tslot = reinterpret_cast<uint64_t*>(p.ctl + ctl::kTauG) + 8 * t;
      if (wg == t) {                     // wait for every participating bound of token t
        const uint64_t* slots = p.tauv + (size_t)t * kMaxWG;
        tm = p.n_part <= 256 ? wait_tagged_min<4>(slots, p.n_part, tag, p.ctl)
                             : wait_tagged_min<16>(slots, p.n_part, tag, p.ctl);
        if (lane == 0) ast64(tslot, ((uint64_t)tag << 32) | tm);
      } else {
        tm = wait_tagged_one(tslot, tag, p.ctl);
      }
    }
    DSA_MARK(p.trace, 5);
    // score >= tau as a float compare (equal keys <=> equal floats, -0 == +0)
    const float tauf = tm ? key_to_float(tm) : -__builtin_inff();
    const int64_t lim64 = p.pos0 + t - c0;
    const int lim = (int)(lim64 < nkeys - 1 ? lim64 : nkeys - 1);      // last visible local index
    uint64_t* dst = p.cand + ((size_t)t * p.nwg + wg) * p.chunk;
    // Lane l takes local positions 64 l .. 64 l + 63 (the chunk holds at most 64 x 64):
    // sixteen 16-byte reads in a lane-rotated order (lanes of different l mod 16 hit
    // different banks) give a 64-bit mask of its visible scores >= tau, one wave scan of
    // the lanes' counts gives its first slot, and a short loop stores its candidates, so
    // they leave in position order.  (The compares are independent, so the pass is short;
    // a pass over 512-position batches with a wave scan each was bound by the latency of
    // its dependent steps.)
    const int pb = 64 * lane;
    // candidates among the kMaxChunk local positions sb .. held at `row`, visible up to
    // local position sb + lims, stored from slot ob on; returns how many
    auto emit = [&](auto guard, const float* row, int sb, int lims, uint32_t ob) -> uint32_t {
      const int nv = lims + 1 - pb;                                       // visible positions of this lane
      uint64_t mk = 0ull;
      if (nv > 0) {
        const float4* r4 = reinterpret_cast<const float4*>(row + pb);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const int cc = (c + lane) & 15;
          float4 v;
          // guarded rows read no float4 that starts past the last visible position
          if constexpr (decltype(guard)::value) {
            const float ninf = -__builtin_inff();
            v = 4 * cc < nv ? r4[cc] : make_float4(ninf, ninf, ninf, ninf);
          } else {
            v = r4[cc];
          }
          const uint32_t nib = (v.x >= tauf ? 1u : 0u) | (v.y >= tauf ? 2u : 0u) | (v.z >= tauf ? 4u : 0u) |
                               (v.w >= tauf ? 8u : 0u);
          mk |= (uint64_t)nib << (4 * cc);
        }
        if (nv < 64) mk &= (1ull << nv) - 1ull;                           // drop positions past lim
      }
      uint32_t mlo = (uint32_t)mk, mhi = (uint32_t)(mk >> 32);
      const uint32_t cnt = (uint32_t)__builtin_popcount(mlo) + (uint32_t)__builtin_popcount(mhi);
      const uint32_t inc = wave_incl_scan(cnt);
      uint32_t o = ob + inc - cnt;
      while ((mlo | mhi) != 0u) {
        int i;
        if (mlo != 0u) { i = __builtin_ctz(mlo); mlo &= mlo - 1u; }
        else { i = 32 + __builtin_ctz(mhi); mhi &= mhi - 1u; }
        ast64(dst + o, ((uint64_t)(uint32_t)(c0 + sb + pb + i) << 32) | order_key(row[pb + i]));
        ++o;
      }
      return (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    };
    uint32_t off = emit(std::false_type{}, sh.sc[t], 0, lim, 0u);
    if constexpr (SPILL) {
      // the chunk's later positions, kMaxChunk at a time, from the spill rows (fused scan)
      // or the input rows (loaded scores), in position order after the LDS part
      for (int sb = kMaxChunk; sb < nkeys; sb += kMaxChunk) {
        const float* row = SRC == 0
            ? p.spill + (size_t)t * p.sstride + (size_t)wg * (p.chunk - kMaxChunk) + (sb - kMaxChunk)
            : p.scores + (size_t)t * p.ld + c0 + sb;
        off += emit(std::true_type{}, row, sb, lim - sb, off);
      }
    }
    vm_wait_all();                       // candidates land before their count
    if (lane == 0) ast64(p.cnt + (size_t)t * p.nwg + wg, ((uint64_t)tag << 32) | off);
    DSA_MARK(p.trace, 6);
  }
  DSA_MARK(p.trace, 7);
  // ---------------- P3: workgroup t selects token t once every count of the token is in
  if (wg < T) resolve_token(p, wg, sh, epoch);
  DSA_MARK(p.trace, 15);
  return true;
}

}  // namespace dsa
