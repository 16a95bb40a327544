// Device-side building blocks shared by the gfx950 kernels: number formats, the
// MFMA operand types, order-preserving keys, block scans and the grid barrier.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

#define DSA_DEV __device__ __forceinline__

constexpr int kHq = 8;       // query heads per GPU share
constexpr int kD = 128;      // head width
constexpr int kHI = 16;      // indexer heads
constexpr int kDI = 64;      // indexer head width
constexpr int kMaxT = 8;     // verify block
constexpr int kMaxTopK = 2048;
constexpr int kHidden = 4096;
constexpr int kNProjDSA = kHq * kD + 2 * kD + kHI * kDI + kDI + kHI;  // 2384
constexpr int kNProjSWA = kHq * kD + 2 * kD;                          // 1280

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

union Frag8 {           // eight bf16 = one MFMA A/B operand of the K=16/K=32 shapes
  bf16x8_t v;
  uint4 u;
  uint32_t w[4];
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Four 16-bit values through the LDS transpose path: within each 16-lane group, lane q
// supplies the 8 bytes at its address and receives element (q & 3) of the values
// supplied by lanes (q >> 2) + 4i, i = 0..3.  With lane q of group g pointing at row
// r0 + (q >> 2), columns c0 + 16 (g & 1) + 4 (q & 3) .. +3 of a row-major bf16 matrix,
// lane l receives rows r0 .. r0 + 3 of column c0 + (l & 31): the K-major layout of a
// 32x32x16 MFMA B operand (the next four rows come from a second read 4 rows further).
DSA_DEV uint2 lds_tr16(const uint8_t* addr) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(reinterpret_cast<uintptr_t>(addr)));
  return __builtin_bit_cast(uint2, r);
}

// ----------------------------------------------------------------------------- formats

DSA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet)
DSA_DEV uint16_t f32_to_bf16(float f) {
  const __bf16 b = (__bf16)f;                 // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

DSA_DEV float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// two fp32 -> (lo, hi) bf16 pair in one word, each rounded to nearest even
DSA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v b = __builtin_convertvector(f32x2v{lo, hi}, bf16x2v);
  return __builtin_bit_cast(uint32_t, b);
}

// OCP e4m3fn code -> fp32, exact (integer construction of the IEEE bits)
DSA_DEV float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t m = c & 7u;
  if (e == 15u && m == 7u) return __uint_as_float(0x7fc00000u | s);
  if (e == 0u) {                       // subnormal: m * 2^-9, exact in fp32
    float v = (float)m * 0x1p-9f;
    return __uint_as_float(__float_as_uint(v) | s);
  }
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// fp32 -> e4m3fn code: nearest, ties to even, saturating at +-448; sign kept (also for 0).
DSA_DEV uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t s = (u >> 24) & 0x80u;
  float a = fminf(fabsf(x), 448.0f);
  uint32_t au = __float_as_uint(a);
  int e = (int)(au >> 23) - 127;       // unbiased exponent of a (a > 0)
  if (a == 0.0f) return s;
  uint32_t code;
  if (e < -6) {
    // subnormal range: quantum 2^-9; a * 2^9 in [0, 8), exact scaling
    float r = a * 512.0f;
    float f = floorf(r);
    float rem = r - f;                 // exact
    uint32_t q = (uint32_t)f;
    if (rem > 0.5f || (rem == 0.5f && (q & 1u))) q += 1u;
    code = q;                          // q == 8 is the smallest normal (code 8) -- consistent
  } else {
    // normal: 3 mantissa bits; round the 23-bit fraction to 3 bits
    uint32_t mant = au & 0x7fffffu;
    uint32_t keep = mant >> 20;
    uint32_t rest = mant & 0xfffffu;
    uint32_t half = 0x80000u;
    uint32_t q = ((uint32_t)(e + 7) << 3) | keep;
    if (rest > half || (rest == half && (q & 1u))) q += 1u;
    code = q;                          // a <= 448 so q <= 126 after rounding
  }
  return s | code;
}

// ------------------------------------------------------------------ W8A8 activations
// Per-token e4m3 quantisation of bf16 activations: codes = e4m3(fp32(y * inv)) with
// inv = fp32(448 / amax) (1 for an all-zero token), dequantisation scale fp32(amax / 448).

// largest magnitude of eight bf16 held as four (lo, hi) pairs
DSA_DEV float amax_bf16x8(const uint32_t y[4]) {
  float m = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(y[q] << 16)), fabsf(__uint_as_float(y[q] & 0xffff0000u))));
  return m;
}

// eight bf16 (four pairs) times inv -> eight e4m3 codes, element i in byte i.  The
// hardware conversion rounds to nearest even; |y * inv| <= fp32(448 (1 + 2^-24)) stays
// below the overflow boundary 464, so every product lands on a finite code.
DSA_DEV uint2 e4m3x8_scaled(const uint32_t y[4], float inv) {
  int w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = y[2 * h], b = y[2 * h + 1];
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(a << 16) * inv,
                                            __uint_as_float(a & 0xffff0000u) * inv, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b << 16) * inv,
                                        __uint_as_float(b & 0xffff0000u) * inv, r, true);
    w[h] = r;
  }
  return make_uint2((uint32_t)w[0], (uint32_t)w[1]);
}

// lane exchange inside rows of 16 lanes (DPP): quad permutations and row rotations
template <int CTRL>
DSA_DEV float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// max / sum over the 16 lanes of a row (quads first, then rotations by 4 and 8); every
// lane ends with the row's maximum; the sum's association depends on the lane, so only
// one fixed lane's sum is used
DSA_DEV float row16_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));      // quad_perm [1,0,3,2]
  v = fmaxf(v, dppf<0x4E>(v));      // quad_perm [2,3,0,1]
  v = fmaxf(v, dppf<0x124>(v));     // row_ror:4
  return fmaxf(v, dppf<0x128>(v));  // row_ror:8
}
// maximum over a whole wave (rows of 16 first, then the four row maxima): wave-uniform
DSA_DEV float wave_max(float v) {
  v = row16_max(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
DSA_DEV float row16_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x124>(v);
  return v + dppf<0x128>(v);
}

// ----------------------------------------------------------------------------- keys

// Order-preserving map fp32 -> uint32 (larger score <=> larger key); -0 maps like +0.
DSA_DEV uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----------------------------------------------------------------------------- scans

// DPP lane exchange of a 32-bit value: `old` where the source lane is outside the row or
// the row is masked off (row shifts, row broadcasts)
template <int CTRL, int ROWMASK = 0xf>
DSA_DEV uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xf, false);
}

// Inclusive prefix sum across one wavefront (64 lanes, all active): row shifts by 1, 2, 4
// and 8 within rows of 16 lanes, then lane 15's total into rows 1 and 3 and lane 31's into
// rows 2 and 3.
DSA_DEV uint32_t wave_incl_scan(uint32_t v) {
  v += dppu<0x111>(v);           // row_shr:1
  v += dppu<0x112>(v);           // row_shr:2
  v += dppu<0x114>(v);           // row_shr:4
  v += dppu<0x118>(v);           // row_shr:8
  v += dppu<0x142, 0xa>(v);      // row_bcast:15
  v += dppu<0x143, 0xc>(v);      // row_bcast:31
  return v;
}

// max / min over the wave (all lanes active; every lane gets the result): rotations
// within rows of 16, then the row-pair and half-wave swaps
DSA_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dppu<0xB1>(v));
  v = max(v, dppu<0x4E>(v));
  v = max(v, dppu<0x124>(v));
  v = max(v, dppu<0x128>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)r[0], (uint32_t)r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}

DSA_DEV uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dppu<0xB1>(v));
  v = min(v, dppu<0x4E>(v));
  v = min(v, dppu<0x124>(v));
  v = min(v, dppu<0x128>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min((uint32_t)r[0], (uint32_t)r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min((uint32_t)q[0], (uint32_t)q[1]);
}

// Exclusive prefix sum across the block; `scratch` holds >= nwaves+1 words of LDS.
// Returns the exclusive prefix; *total receives the block sum.  All threads must call.
template <int NT>
DSA_DEV uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane == 63) scratch[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t t = (lane < NW) ? scratch[lane] : 0u;
    uint32_t ti = wave_incl_scan(t);
    if (lane < NW) scratch[lane] = ti - t;   // exclusive wave offsets
    if (lane == NW - 1) scratch[NW] = ti;
  }
  __syncthreads();
  uint32_t res = scratch[wid] + inc - v;
  *total = scratch[NW];
  __syncthreads();
  return res;
}

template <int NT>
DSA_DEV uint32_t block_max_u32(uint32_t v, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = max(r, scratch[i]);
  __syncthreads();
  return r;
}

// minimum and maximum over the block in one exchange (scratch holds 2 * NT / 64 words)
template <int NT>
DSA_DEV void block_minmax_u32(uint32_t& mn, uint32_t& mx, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  const uint32_t a = wave_min_u32(mn), b = wave_max_u32(mx);
  if ((threadIdx.x & 63) == 0) {
    scratch[threadIdx.x >> 6] = a;
    scratch[NW + (threadIdx.x >> 6)] = b;
  }
  __syncthreads();
  uint32_t r0 = scratch[0], r1 = scratch[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    r0 = min(r0, scratch[i]);
    r1 = max(r1, scratch[NW + i]);
  }
  __syncthreads();
  mn = r0;
  mx = r1;
}

template <int NT>
DSA_DEV uint32_t block_min_u32(uint32_t v, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  v = wave_min_u32(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = min(r, scratch[i]);
  __syncthreads();
  return r;
}

// ----------------------------------------------------------------------------- coherent access

// Data that crosses workgroups inside one launch is written and read only through these
// agent-scope relaxed atomics (sc1 loads/stores on gfx950: coherent across the XCDs' L2s
// without writing back or invalidating whole caches).  A producer orders its stores
// before a later signal with vm_wait_all() (all of its own vector memory operations done).
DSA_DEV uint32_t ald(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV uint64_t ald64(const uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV float aldf(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV void ast(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV void ast64(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV void astf(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV uint32_t aadd(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV uint32_t amax(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DSA_DEV void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Control block at the start of every workspace (uint32 index; every polled word on its
// own 256-byte line).  The launch counter and the sticky error word share one 8-byte
// word so a launch reads both with one load.
namespace ctl {
constexpr int kEpoch = 768;      // launch counter (tags of the tagged slots)
constexpr int kError = 769;      // sticky error word (1 = a wait inside a launch gave up)
constexpr int kDone = 1024;      // [8] per-token completion counters, stride 64
constexpr int kTauG = 2048;      // [8] tagged slots (64-bit, stride 16 words): per-token tau
constexpr int kWords = 3072;
constexpr size_t kBytes = 16384;
}  // namespace ctl

// Phase timestamps (100 MHz real-time counter) for profiling builds only (-DDSA_TRACE):
// thread 0 of each workgroup records slot `s` (< 16) of its row in a caller buffer.
#ifdef DSA_TRACE
#define DSA_MARK(buf, s) \
  do { if ((buf) && threadIdx.x == 0) (buf)[blockIdx.x * 16 + (s)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#define DSA_MARK_CLK(buf, s) \
  do { if ((buf) && threadIdx.x == 0) (buf)[blockIdx.x * 16 + (s)] = __builtin_amdgcn_s_memtime(); } while (0)
#else
#define DSA_MARK(buf, s) do { } while (0)
#define DSA_MARK_CLK(buf, s) do { } while (0)
#endif

constexpr uint64_t kSpinLimit = 20000000ull;   // 0.2 s of the 100 MHz real-time counter

// Cross-workgroup hand-offs inside one launch use tagged slots instead of barriers: a
// producer writes (tag << 32 | value) into its own 64-bit slot after its data has landed,
// and a consumer polls the slots it needs until all carry the launch's tag, receiving the
// values with the same loads.  The tag is a launch counter + 1: the counter is read at
// kernel start and advanced by one workgroup once every workgroup has published (so
// every read of it has completed).  It runs through [0, 2^31) and wraps, so a tag is
// never 0 (the value of a cleared workspace).
DSA_DEV uint32_t next_epoch(uint32_t e) { return (e + 1u) & 0x7fffffffu; }

// Wait until one tagged slot carries `tag` and return its value (the wave polls one
// address: one load per round).  A wait longer than kSpinLimit sets the sticky error word
// and gives up, so a launch whose workgroups are not all resident ends instead of hanging.
DSA_DEV uint32_t wait_tagged_one(const uint64_t* slot, uint32_t tag, uint32_t* ctl_words) {
  uint64_t v = ald64(slot);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while ((uint32_t)(v >> 32) != tag) {
    __builtin_amdgcn_s_sleep(1);
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
      if ((threadIdx.x & 63) == 0) ast(ctl_words + ctl::kError, 1u);
      break;
    }
    v = ald64(slot);
  }
  return (uint32_t)v;
}

// N tagged words addr(0 .. N-1) loaded together, then the ones not yet carrying `tag`
// reloaded until all do; the low halves into val.  Bounded: the wait gives up after
// kSpinLimit, or as soon as the workspace's error word is set (another wait of the launch
// gave up), sets the error word and returns false.
template <int N, typename F>
DSA_DEV bool poll_words(F addr, uint32_t tag, uint32_t (&val)[N], uint32_t* ctl_words) {
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = ald64(addr(i));
  bool ok = true;
#pragma unroll
  for (int i = 0; i < N; ++i) ok = ok & ((uint32_t)(v[i] >> 32) == tag);
  if (!ok) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (!ok) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit || ald(ctl_words + ctl::kError) != 0u) {
        ast(ctl_words + ctl::kError, 1u);
        break;
      }
#pragma unroll
      for (int i = 0; i < N; ++i)
        if ((uint32_t)(v[i] >> 32) != tag) v[i] = ald64(addr(i));
      ok = true;
#pragma unroll
      for (int i = 0; i < N; ++i) ok = ok & ((uint32_t)(v[i] >> 32) == tag);
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) val[i] = (uint32_t)v[i];
  return ok;
}

// Wave-wide wait for slots[0 .. n) (n >= 1, n <= 64 * N) to carry `tag`; returns the
// minimum of their values.  After the first round only the slots still without the tag
// are read again.  Bounded like wait_tagged_one.
template <int N>
DSA_DEV uint32_t wait_tagged_min(const uint64_t* slots, int n, uint32_t tag, uint32_t* ctl_words) {
  const int lane = threadIdx.x & 63;
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int w = lane + 64 * i;
    v[i] = ald64(slots + (w < n ? w : n - 1));
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok & ((uint32_t)(v[i] >> 32) == tag);
    if (__ballot(!ok) == 0ull) break;
    __builtin_amdgcn_s_sleep(1);
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
      if (lane == 0) ast(ctl_words + ctl::kError, 1u);
      break;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {        // only the slots still without the tag
      const int w = lane + 64 * i;
      if ((uint32_t)(v[i] >> 32) != tag) v[i] = ald64(slots + (w < n ? w : n - 1));
    }
  }
  uint32_t m = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < N; ++i) m = min(m, (lane + 64 * i < n) ? (uint32_t)v[i] : 0xffffffffu);
  return wave_min_u32(m);
}

}  // namespace dsa
