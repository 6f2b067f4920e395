// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace parallax {

struct DecodeArgs {
  const void* q;
  const void* rho;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  float* out;
  void* ws;        // partial records [B, H_q, num_splits, 2d + 4] fp32
  void* counters;  // arrival counters (fused merge), or null for the two-phase form
  int B, H_q, H_kv, G, d, S_max;
  int num_splits, chunk;
  float scale;
  bool f32;
};

struct PrefillArgs {
  const void* q;
  const void* rho;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* past_lens;  // null: no past (plain causal prefill)
  float* out;
  int B, H_q, H_kv, G, d, T, S_max;
  float scale;
};

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

}  // namespace parallax
