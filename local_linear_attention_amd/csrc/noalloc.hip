// Allocation-free decode: parallax_decode with its partial records and
// arrival counters in a scratch array the library holds on each device, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. In host
// code its name is only a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress and that address is what the
// kernels receive. Layout: arrival counters first (a fixed place, so that the
// zeros each call leaves behind are where the next call looks for them, at
// any size), then the partial records.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "parallax.h"

namespace parallax {
namespace {

constexpr size_t kScratchBytes = PARALLAX_NOALLOC_SCRATCH_BYTES;
constexpr size_t kCounterBytes = PARALLAX_NOALLOC_COUNTER_BYTES;
static_assert(kCounterBytes % 256 == 0 && kCounterBytes < kScratchBytes, "scratch layout");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device (null: not yet set up)

// Zeroes n 32-bit words (a fill kernel rather than a memset node, so that the
// clear can also sit in a captured graph).
__global__ __launch_bounds__(256) void zero_words(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// Device address of this device's scratch. On the first call for a device
// (that device current) it looks the address up and clears the counters on
// `stream`; the decode launched after it on the same stream is ordered
// behind the clear.
parallax_status_t scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PARALLAX_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PARALLAX_ERR_HIP;
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       kCounterBytes / sizeof(uint32_t));
    if (hipGetLastError() != hipSuccess) return PARALLAX_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PARALLAX_OK;
}

}  // namespace
}  // namespace parallax

extern "C" parallax_status_t parallax_decode_noalloc(const void* q, const void* rho,
                                                     const void* k_cache, const void* v_cache,
                                                     const int32_t* seq_lens, float* out, int B,
                                                     int H_q, int H_kv, int d, int S_max,
                                                     float scale, parallax_dtype_t dtype,
                                                     int num_splits, void* stream) {
  return parallax::decode_in_scratch(q, rho, k_cache, v_cache, seq_lens, out, B, H_q, H_kv, d,
                                     S_max, scale, dtype, num_splits,
                                     parallax::scratch_on_current_device, parallax::kScratchBytes,
                                     parallax::kCounterBytes, stream);
}
