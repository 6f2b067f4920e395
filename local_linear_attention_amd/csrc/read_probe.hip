// Plain streaming read, a measurement reference for the decode kernel's KV
// stream (not part of the method): every 16-byte word of two buffers is read
// exactly once and folded by XOR into a sink array, so the reads cannot be
// dropped and the result can be checked on the host.
//
// Workgroups of 256 threads, about two per compute unit like the decode
// launch; workgroup w streams one contiguous share of the two buffers (taken
// as one sequence of words), each thread keeping 8 non-temporal 16-byte loads
// in flight. Each workgroup folds its XOR into word w mod sink_words of the
// sink with one atomic: a single shared word would serialise the atomics of
// every workgroup at the end of the launch.

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const i32x4* __restrict__ a,
                                                              const i32x4* __restrict__ b,
                                                              unsigned long long n16,
                                                              uint32_t* __restrict__ sink,
                                                              unsigned sink_words) {
  const unsigned long long total = 2ull * n16;
  const unsigned long long per = (total + gridDim.x - 1) / gridDim.x;
  const unsigned long long lo = (unsigned long long)blockIdx.x * per;
  const unsigned long long hi = lo + per < total ? lo + per : total;
  uint32_t x = 0;
  for (unsigned long long i = lo + threadIdx.x; i < hi; i += (unsigned long long)kThreads * kUnroll) {
    i32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const unsigned long long j = i + (unsigned long long)kThreads * u;
      v[u] = j < hi ? __builtin_nontemporal_load(j < n16 ? a + j : b + (j - n16)) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x ^= __shfl_xor(x, s);
  __shared__ uint32_t wave_x[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) y ^= wave_x[w];
    atomicXor(sink + blockIdx.x % sink_words, y);
  }
}

}  // namespace

hipError_t launch_read_probe(const void* a, const void* b, size_t bytes_each, uint32_t* sink,
                             unsigned sink_words, int workgroups, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kThreads), 0, st,
                     static_cast<const i32x4*>(a), static_cast<const i32x4*>(b),
                     (unsigned long long)(bytes_each / 16), sink, sink_words);
  return hipGetLastError();
}

}  // namespace parallax
