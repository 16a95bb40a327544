// Measurement helper, built as its own library (libdsa_read_ceiling.so) and used by the
// benchmark only; it is no step of the method and not part of libdsa.so.
//
// Streaming read of a device buffer: the measured HBM read ceiling that the kernels'
// achieved bandwidth is compared with.  One 1024-thread workgroup per compute unit
// reads a contiguous slice with four 16-byte loads in flight per thread (64 KiB per
// CU), folds the words with xor and writes one word per workgroup, so the write
// traffic is negligible and the loads cannot be elided.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kSrThreads = 1024;
constexpr int kSrUnroll = 4;

__global__ void __launch_bounds__(kSrThreads) stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                                 size_t per, uint32_t* sink) {
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  size_t i = beg + threadIdx.x;
  // full rounds: every load of the round is in range, so none is conditional
  for (; i + (size_t)(kSrUnroll - 1) * kSrThreads < end; i += (size_t)kSrUnroll * kSrThreads) {
    uint4 v[kSrUnroll];
#pragma unroll
    for (int u = 0; u < kSrUnroll; ++u) v[u] = src[i + (size_t)u * kSrThreads];
#pragma unroll
    for (int u = 0; u < kSrUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kSrThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
  __shared__ uint32_t part[kSrThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int w = 0; w < kSrThreads / 64; ++w) a ^= part[w];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

// Reads `bytes` (a multiple of 16, src 16-byte aligned) as a plain stream with one
// workgroup per compute unit (at most 1024) and writes an xor fold of it to
// sink[0 .. workgroups) (caller-owned, at least 1024 uint32 words on the device).
// Returns 0, or -1 for bad arguments, or the HIP error code of the launch.
extern "C" int dsa_read_ceiling_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15u) || (bytes & 15u) || bytes == 0) return -1;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipGetLastError();
  const int nblocks = ncu < 1024 ? ncu : 1024;
  const size_t n16 = bytes / 16;
  const size_t per = (n16 + nblocks - 1) / nblocks;
  hipLaunchKernelGGL(stream_read_kernel, dim3(nblocks), dim3(kSrThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(src), n16, per, sink);
  return (int)hipGetLastError();
}
