// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "parallax.h"

namespace parallax {

struct DecodeArgs {
  const void* q;
  const void* rho;
  const void* k;
  const void* v;
  const int32_t* seq_lens;   // key counts, or chunk lengths with past_lens
  const int32_t* past_lens;  // several tokens per sequence: cached lengths; else null
  float* out;
  void* ws;        // partial records [B, H_q, num_splits, 2d + 4] fp32
  void* counters;  // arrival counters (fused merge), or null for the two-phase form
  int B, H_q, H_kv, G, d, S_max;
  int num_splits, chunk;
  int ntok;  // tokens per sequence (H_q and G above count (head, token) pairs)
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
  float* mu_out;  // training mode: mu_v [B, H_q, T, d] fp32, else null
  void* stats;    // training mode: [B, H_q, T] x (lse2, c, rbar - c, 0) fp32, else null
  int B, H_q, H_kv, G, d, T, S_max;
  float scale;
};

// Causal prefill backward. The workspace holds dO split into bf16 high and
// low parts ([B, H_q, T, d] each) and per-row (G, Dt) = (dO.mu_v, dO.out).
struct BwdArgs {
  const void* q;
  const void* rho;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const float* out;
  const float* mu;
  const float4* stats;
  const float* dout;
  float* dq;
  float* drho;
  float* dk;
  float* dv;
  __bf16* dhi;
  __bf16* dlo;
  float2* gd;
  int B, H_q, H_kv, G, d, T, S_max;
  float scale, scale_log2;
};

// Fused q, k, v, rho projection of x [B T, d_model] by the packed weight
// W [(2 H_q + 2 H_kv) d, d_model] (rows W_Q, W_K, W_V, W_R).
struct ProjArgs {
  const void* x;
  const void* w;
  void* q;
  void* k;
  void* v;
  void* rho;
  const int32_t* past_lens;  // k, v rows written at past_lens[b] + t (null: 0)
  int B, T, d_model, H_q, H_kv, d, S_max;
};

// Query heads one decode workgroup serves: 8 (two probe tiles) when a KV
// head has more than 4, else 4. The split plan counts workgroup streams of
// this many heads.
inline int decode_heads_per_workgroup(int G) { return G > 4 ? 8 : 4; }

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t st);

// parallax_decode with its partial records and arrival counters in a
// scratch region supplied by `get_scratch` after every argument check has
// passed (defined in api.cpp; used by the allocation-free entry point).
typedef parallax_status_t (*ScratchFn)(hipStream_t stream, void** base);
parallax_status_t decode_in_scratch(const void* q, const void* rho, const void* k_cache,
                                    const void* v_cache, const int32_t* seq_lens, float* out, int B,
                                    int H_q, int H_kv, int d, int S_max, float scale,
                                    parallax_dtype_t dtype, int num_splits, ScratchFn get_scratch,
                                    size_t scratch_bytes, size_t counter_bytes, void* stream);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_backward(const BwdArgs& a, hipStream_t st);
hipError_t launch_projection(const ProjArgs& a, hipStream_t st);
hipError_t launch_read_probe(const void* a, const void* b, size_t bytes_each, uint32_t* sink,
                             unsigned sink_words, int workgroups, hipStream_t st);

}  // namespace parallax
