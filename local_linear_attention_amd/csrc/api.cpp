// extern "C" entry points of libparallax (declared in include/parallax.h).
// Host code only: argument checks, split planning and kernel launches on the
// caller's stream. No allocation, no synchronisation, no exceptions across
// the boundary.

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "parallax.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device, queried once per device.
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int round_up(long long x, int m) { return (int)(((x + m - 1) / m) * m); }

constexpr int kChunkQuantum = 128;  // keys per workgroup pass (4 waves x 32 keys)
constexpr int kMaxAutoSplits = 32;  // automatic plans use at most this many splits

// Split plan: chunk (keys per workgroup, multiple of 128) and split count.
parallax_status_t plan(int B, int H_q, int H_kv, int d, int S_max, int requested, int* ns_out,
                       int* chunk_out) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || S_max <= 0 || H_q % H_kv != 0)
    return PARALLAX_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return PARALLAX_ERR_UNSUPPORTED;
  // the padded key range must stay an int
  if (S_max > INT_MAX - kChunkQuantum) return PARALLAX_ERR_UNSUPPORTED;
  const int G = H_q / H_kv;
  const int hw = parallax::decode_heads_per_workgroup(G);
  const long long groups = ((long long)G + hw - 1) / hw;
  // H_kv * groups <= H_q / hw + H_kv < 2^32, so this product stays below 2^63
  const long long streams = (long long)B * ((long long)H_kv * groups);
  const int full = round_up(S_max, kChunkQuantum);
  int chunk;
  if (requested > 0) {
    chunk = round_up((S_max + (long long)requested - 1) / requested, kChunkQuantum);
  } else {
    const int cus = cu_count();
    if (cus <= 0) return PARALLAX_ERR_HIP;
    // About one workgroup per compute unit over the padded key range (a
    // second workgroup on a compute unit trails the first: gqa-decode, 8 x 4096
    // keys, takes 25.4 us at 4 splits against 26.3 at 8), with chunks of
    // 128..2048 keys (the cap keeps ragged batches balanced), at most 32 splits
    // per stream (the fused merge reads every split's record), and at most 16
    // splits when the chunks come out shorter than 512 keys: there each
    // workgroup streams for so short a time that the merge's record reads
    // decide, while a few more splits still cut the latency of small batches
    // (one 1024-key sequence: 2 splits 11.0 us, 8 splits 7.5 us).
    // For bf16 at d = 64 the workgroup has 8 waves instead of 4 (its rows
    // are half as long), and one per compute unit is again best (gqa shape
    // at d = 64: 4 splits 15.7 us, 8 splits 16.4 us, 2 splits 16.8 us).
    const long long target = (long long)cus;
    // streams beyond 2048 target's worth give the 2048-key cap anyway; capping
    // them keeps the product inside 64 bits
    const long long st_c = streams < target * 2048 ? streams : target * 2048;
    long long want = ((long long)S_max * st_c + target - 1) / target;
    if (want > 2048) want = 2048;  // the cap below, applied before the narrowing to int
    chunk = round_up(want, kChunkQuantum);
    if (chunk < kChunkQuantum) chunk = kChunkQuantum;
    if (chunk > 2048) chunk = 2048;
    const int min_chunk = round_up((S_max + kMaxAutoSplits - 1) / kMaxAutoSplits, kChunkQuantum);
    if (chunk < min_chunk) chunk = min_chunk;
    if (chunk < 512) {
      const int min_small = round_up((S_max + 15) / 16, kChunkQuantum);
      if (chunk < min_small) chunk = min_small;
    }
  }
  if (chunk > full) chunk = full;
  const int ns = (int)(((long long)S_max + chunk - 1) / chunk);
  if (ns_out) *ns_out = ns;
  if (chunk_out) *chunk_out = chunk;
  return PARALLAX_OK;
}

// Workspaces of 2^62 bytes or more are refused (no device holds one): every
// size below is then exact in size_t.
constexpr unsigned long long kMaxWorkspace = 1ull << 62;

// Whether the partial records and counters of a plan stay below kMaxWorkspace.
bool workspace_fits(int B, int H_q, int d, int ns) {
  const unsigned __int128 rec = (unsigned __int128)(unsigned)B * (unsigned)H_q * (unsigned)ns *
                                (unsigned)(2 * d + 4) * sizeof(float);
  const unsigned __int128 ctr = (unsigned __int128)(unsigned)B * (unsigned)H_q * sizeof(uint32_t) + 16;
  return rec + ctr < kMaxWorkspace;
}

size_t records_bytes(int B, int H_q, int d, int ns) {
  return (size_t)B * H_q * ns * (size_t)(2 * d + 4) * sizeof(float);
}

// Partial records, then one 32-bit arrival counter per (b, query head) (an
// upper bound on the (b, KV head, head group) streams), rounded to 16 bytes.
// 0 for a one-split plan, a bad shape or a workspace past kMaxWorkspace.
size_t workspace_bytes_for(int B, int H_q, int d, int ns) {
  if (B <= 0 || H_q <= 0 || d <= 0 || ns <= 1 || !workspace_fits(B, H_q, d, ns)) return 0;
  const size_t ctr = ((size_t)B * H_q * sizeof(uint32_t) + 15) / 16 * 16;
  return records_bytes(B, H_q, d, ns) + ctr;
}

struct Checked {
  parallax::DecodeArgs a;
  size_t ws_need;
};

parallax_status_t check_decode(const void* q, const void* rho, const void* k, const void* v,
                               const int32_t* seq_lens, float* out, bool need_out, int B,
                               int H_q, int H_kv, int d, int S_max, float scale,
                               parallax_dtype_t dtype, int num_splits, void* ws,
                               size_t ws_bytes, Checked* c, bool check_ws = true) {
  if (!q || !rho || !k || !v || !seq_lens) return PARALLAX_ERR_NULL_POINTER;
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || S_max <= 0 || num_splits < 0 ||
      H_q % H_kv != 0)
    return PARALLAX_ERR_BAD_SHAPE;
  if (dtype != PARALLAX_BF16 && dtype != PARALLAX_F32) return PARALLAX_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return PARALLAX_ERR_UNSUPPORTED;
  const int G = H_q / H_kv;
  const long long esz = dtype == PARALLAX_F32 ? 4 : 2;
  if (((long long)S_max + 64) * d * esz >= (1LL << 31)) return PARALLAX_ERR_UNSUPPORTED;
  // one sequence's queries under 2 GiB: keeps head counts and the grid well inside int
  if ((long long)H_q * d * esz >= (1LL << 31)) return PARALLAX_ERR_UNSUPPORTED;
  if (B > 65535) return PARALLAX_ERR_UNSUPPORTED;  // grid y
  if (!std::isfinite(scale)) return PARALLAX_ERR_BAD_SHAPE;  // NaN or infinite scale
  if (!aligned16(q) || !aligned16(rho) || !aligned16(k) || !aligned16(v) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return PARALLAX_ERR_MISALIGNED;
  int ns = 0, chunk = 0;
  parallax_status_t st = plan(B, H_q, H_kv, d, S_max, num_splits, &ns, &chunk);
  if (st != PARALLAX_OK) return st;
  if (ns > 65535) return PARALLAX_ERR_UNSUPPORTED;  // grid z
  if (ns > 1 && !workspace_fits(B, H_q, d, ns)) return PARALLAX_ERR_UNSUPPORTED;
  const bool direct = (ns == 1);
  if ((direct || need_out) && !out) return PARALLAX_ERR_NULL_POINTER;
  if (out && !aligned16(out)) return PARALLAX_ERR_MISALIGNED;
  const size_t need = workspace_bytes_for(B, H_q, d, ns);
  if (need > 0 && check_ws) {
    if (!ws || ws_bytes < need) return PARALLAX_ERR_WORKSPACE;
    if (!aligned16(ws)) return PARALLAX_ERR_MISALIGNED;
  }
  c->ws_need = need;
  void* counters = nullptr;
  if (need > 0 && need_out && ws)
    counters = static_cast<char*>(ws) + records_bytes(B, H_q, d, ns);
  c->a = parallax::DecodeArgs{q, rho, k, v, seq_lens, nullptr, out, ws, counters, B, H_q, H_kv,
                              G, d, S_max, ns, chunk, 1, scale, dtype == PARALLAX_F32};
  return PARALLAX_OK;
}

parallax_status_t hip_status(hipError_t e) { return e == hipSuccess ? PARALLAX_OK : PARALLAX_ERR_HIP; }

}  // namespace

namespace parallax {

// parallax_decode with the partial records and arrival counters in a scratch
// region that `get_scratch` supplies: counters at its start (counter_bytes),
// records after them. Every argument check runs first; `get_scratch` is
// called (and may launch its own set-up on `stream`) only when the call will
// launch, and only when the plan has several splits. PARALLAX_ERR_TOO_LARGE
// when the plan's records or counters exceed their part of the region.
parallax_status_t decode_in_scratch(const void* q, const void* rho, const void* k_cache,
                                    const void* v_cache, const int32_t* seq_lens, float* out, int B,
                                    int H_q, int H_kv, int d, int S_max, float scale,
                                    parallax_dtype_t dtype, int num_splits, ScratchFn get_scratch,
                                    size_t scratch_bytes, size_t counter_bytes, void* stream) {
  try {
    Checked c;
    parallax_status_t st = check_decode(q, rho, k_cache, v_cache, seq_lens, out, true, B, H_q, H_kv,
                                        d, S_max, scale, dtype, num_splits, nullptr, 0, &c, false);
    if (st != PARALLAX_OK) return st;
    if (c.ws_need > 0) {
      if ((size_t)B * H_q * sizeof(uint32_t) > counter_bytes ||
          records_bytes(B, H_q, d, c.a.num_splits) > scratch_bytes - counter_bytes)
        return PARALLAX_ERR_TOO_LARGE;
      void* base = nullptr;
      st = get_scratch(static_cast<hipStream_t>(stream), &base);
      if (st != PARALLAX_OK) return st;
      c.a.counters = base;
      c.a.ws = static_cast<char*>(base) + counter_bytes;
    }
    return hip_status(launch_decode_partial(c.a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

}  // namespace parallax

extern "C" {

int parallax_abi_version(void) { return PARALLAX_ABI_VERSION; }

const char* parallax_status_string(parallax_status_t s) {
  switch (s) {
    case PARALLAX_OK: return "PARALLAX_OK";
    case PARALLAX_ERR_NULL_POINTER: return "PARALLAX_ERR_NULL_POINTER: a required pointer is NULL";
    case PARALLAX_ERR_BAD_SHAPE: return "PARALLAX_ERR_BAD_SHAPE: invalid sizes";
    case PARALLAX_ERR_UNSUPPORTED: return "PARALLAX_ERR_UNSUPPORTED: head dim, group size, dtype or size not built";
    case PARALLAX_ERR_MISALIGNED: return "PARALLAX_ERR_MISALIGNED: a tensor pointer is not 16-byte aligned";
    case PARALLAX_ERR_WORKSPACE: return "PARALLAX_ERR_WORKSPACE: workspace missing or too small";
    case PARALLAX_ERR_HIP: return "PARALLAX_ERR_HIP: HIP runtime or launch failure";
    case PARALLAX_ERR_TOO_LARGE:
      return "PARALLAX_ERR_TOO_LARGE: the sizes exceed the built-in scratch of parallax_decode_noalloc";
  }
  return "unknown parallax status";
}

parallax_status_t parallax_decode_plan(int B, int H_q, int H_kv, int d, int S_max, int requested,
                                       int* num_splits, int* chunk) {
  try {
    if (requested < 0) return PARALLAX_ERR_BAD_SHAPE;
    return plan(B, H_q, H_kv, d, S_max, requested, num_splits, chunk);
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

size_t parallax_decode_workspace_size(int B, int H_q, int d, int num_splits) {
  return workspace_bytes_for(B, H_q, d, num_splits);
}

parallax_status_t parallax_decode_partial(const void* q, const void* rho, const void* k_cache,
                                          const void* v_cache, const int32_t* seq_lens,
                                          float* out, int B, int H_q, int H_kv, int d,
                                          int S_max, float scale, parallax_dtype_t dtype,
                                          int num_splits, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  try {
    Checked c;
    parallax_status_t st = check_decode(q, rho, k_cache, v_cache, seq_lens, out, false, B, H_q,
                                        H_kv, d, S_max, scale, dtype, num_splits, workspace,
                                        workspace_bytes, &c);
    if (st != PARALLAX_OK) return st;
    return hip_status(parallax::launch_decode_partial(c.a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

parallax_status_t parallax_decode_combine(const int32_t* seq_lens, float* out, int B, int H_q,
                                          int H_kv, int d, int S_max, int num_splits,
                                          const void* workspace, size_t workspace_bytes,
                                          void* stream) {
  try {
    if (!seq_lens || !out) return PARALLAX_ERR_NULL_POINTER;
    if (B <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || S_max <= 0 || num_splits < 0 ||
        H_q % H_kv != 0)
      return PARALLAX_ERR_BAD_SHAPE;
    if (d != 64 && d != 128) return PARALLAX_ERR_UNSUPPORTED;
    if (!aligned16(out)) return PARALLAX_ERR_MISALIGNED;
    int ns = 0, chunk = 0;
    parallax_status_t st = plan(B, H_q, H_kv, d, S_max, num_splits, &ns, &chunk);
    if (st != PARALLAX_OK) return st;
    if (ns == 1) return PARALLAX_OK;
    if (!workspace_fits(B, H_q, d, ns)) return PARALLAX_ERR_UNSUPPORTED;
    const size_t need = workspace_bytes_for(B, H_q, d, ns);
    if (!workspace || workspace_bytes < need) return PARALLAX_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PARALLAX_ERR_MISALIGNED;
    parallax::DecodeArgs a{};
    a.seq_lens = seq_lens;
    a.out = out;
    a.ws = const_cast<void*>(workspace);
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = H_q / H_kv;
    a.d = d;
    a.S_max = S_max;
    a.num_splits = ns;
    a.chunk = chunk;
    return hip_status(parallax::launch_decode_combine(a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

parallax_status_t parallax_decode(const void* q, const void* rho, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens, float* out,
                                  int B, int H_q, int H_kv, int d, int S_max, float scale,
                                  parallax_dtype_t dtype, int num_splits, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  try {
    Checked c;
    parallax_status_t st = check_decode(q, rho, k_cache, v_cache, seq_lens, out, true, B, H_q,
                                        H_kv, d, S_max, scale, dtype, num_splits, workspace,
                                        workspace_bytes, &c);
    if (st != PARALLAX_OK) return st;
    // one launch: with several splits the last workgroup of each stream merges
    return hip_status(parallax::launch_decode_partial(c.a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

parallax_status_t parallax_decode_tokens(const void* q, const void* rho, const void* k_cache,
                                         const void* v_cache, const int32_t* past_lens,
                                         const int32_t* chunk_lens, float* out, int B, int H_q,
                                         int H_kv, int d, int T, int S_max, float scale,
                                         parallax_dtype_t dtype, int num_splits,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!past_lens) return PARALLAX_ERR_NULL_POINTER;
    if (T <= 0 || H_q <= 0 || H_kv <= 0 || S_max <= 0 || T > S_max || H_q % H_kv != 0)
      return PARALLAX_ERR_BAD_SHAPE;
    if ((long long)H_q * T > INT_MAX / 2) return PARALLAX_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(past_lens) & 3u) return PARALLAX_ERR_MISALIGNED;
    // every (head, token) pair is one query of the decode kernel
    Checked c;
    parallax_status_t st = check_decode(q, rho, k_cache, v_cache, chunk_lens, out, true, B,
                                        H_q * T, H_kv, d, S_max, scale, dtype, num_splits,
                                        workspace, workspace_bytes, &c);
    if (st != PARALLAX_OK) return st;
    c.a.past_lens = past_lens;
    c.a.ntok = T;
    return hip_status(parallax::launch_decode_partial(c.a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

}  // extern "C"

namespace {

parallax_status_t prefill_common(const void* q, const void* rho, const void* k, const void* v,
                                 const int32_t* seq_lens, const int32_t* past_lens, float* out,
                                 int B, int H_q, int H_kv, int d, int T, int S_max, float scale,
                                 parallax_dtype_t dtype, void* stream) {
  if (!q || !rho || !k || !v || !seq_lens || !out) return PARALLAX_ERR_NULL_POINTER;
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || T <= 0 || S_max <= 0 || T > S_max ||
      H_q % H_kv != 0)
    return PARALLAX_ERR_BAD_SHAPE;
  if (dtype != PARALLAX_BF16) return PARALLAX_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return PARALLAX_ERR_UNSUPPORTED;
  if (((long long)S_max + 256) * d * 2 >= (1LL << 31) ||
      ((long long)T + 256) * d * 2 >= (1LL << 31))
    return PARALLAX_ERR_UNSUPPORTED;
  if (B > 65535 || H_q > 65535) return PARALLAX_ERR_UNSUPPORTED;  // grid y, z limits
  if (!std::isfinite(scale)) return PARALLAX_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(rho) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(past_lens) & 3u))
    return PARALLAX_ERR_MISALIGNED;
  parallax::PrefillArgs a{q,   rho,  k,          v, seq_lens, past_lens, out, nullptr, nullptr, B,
                          H_q, H_kv, H_q / H_kv, d, T,        S_max,     scale};
  return hip_status(parallax::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

parallax_status_t parallax_prefill(const void* q, const void* rho, const void* k, const void* v,
                                   const int32_t* seq_lens, float* out, int B, int H_q, int H_kv,
                                   int d, int T, int S_max, float scale, parallax_dtype_t dtype,
                                   void* stream) {
  try {
    return prefill_common(q, rho, k, v, seq_lens, nullptr, out, B, H_q, H_kv, d, T, S_max, scale,
                          dtype, stream);
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

parallax_status_t parallax_prefill_chunked(const void* q, const void* rho, const void* k_cache,
                                           const void* v_cache, const int32_t* past_lens,
                                           const int32_t* chunk_lens, float* out, int B, int H_q,
                                           int H_kv, int d, int T, int S_max, float scale,
                                           parallax_dtype_t dtype, void* stream) {
  try {
    if (!past_lens) return PARALLAX_ERR_NULL_POINTER;
    return prefill_common(q, rho, k_cache, v_cache, chunk_lens, past_lens, out, B, H_q, H_kv, d,
                          T, S_max, scale, dtype, stream);
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

}  // extern "C"

namespace {

// 0 for a shape the backward refuses (the bounds of check_prefill_shape, under
// which every size here is exact).
size_t bwd_workspace_bytes(int B, int H_q, int T, int d) {
  if (B <= 0 || H_q <= 0 || T <= 0 || (d != 64 && d != 128) || B > 65535 || H_q > 65535 ||
      ((long long)T + 256) * d * 4 >= (1LL << 31))
    return 0;
  const size_t rows = (size_t)B * H_q * T;
  const size_t half = rows * d * 2;          // one bf16 copy of dO
  return ((2 * half + rows * 8) + 15) / 16 * 16;
}

// Shape and pointer checks shared by the training forward and the backward.
parallax_status_t check_prefill_shape(int B, int H_q, int H_kv, int d, int T, int S_max,
                                      float scale, parallax_dtype_t dtype) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || T <= 0 || S_max <= 0 || T > S_max ||
      H_q % H_kv != 0)
    return PARALLAX_ERR_BAD_SHAPE;
  if (dtype != PARALLAX_BF16) return PARALLAX_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return PARALLAX_ERR_UNSUPPORTED;
  if (((long long)S_max + 256) * d * 4 >= (1LL << 31) || ((long long)T + 256) * d * 4 >= (1LL << 31))
    return PARALLAX_ERR_UNSUPPORTED;
  if (B > 65535 || H_q > 65535) return PARALLAX_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PARALLAX_ERR_BAD_SHAPE;
  return PARALLAX_OK;
}

}  // namespace

extern "C" {

parallax_status_t parallax_prefill_train(const void* q, const void* rho, const void* k,
                                         const void* v, const int32_t* seq_lens, float* out,
                                         float* mu_v, float* stats, int B, int H_q, int H_kv,
                                         int d, int T, int S_max, float scale,
                                         parallax_dtype_t dtype, void* stream) {
  try {
    if (!q || !rho || !k || !v || !seq_lens || !out || !mu_v || !stats)
      return PARALLAX_ERR_NULL_POINTER;
    const parallax_status_t st = check_prefill_shape(B, H_q, H_kv, d, T, S_max, scale, dtype);
    if (st != PARALLAX_OK) return st;
    if (!aligned16(q) || !aligned16(rho) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(mu_v) || !aligned16(stats) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
      return PARALLAX_ERR_MISALIGNED;
    parallax::PrefillArgs a{q,   rho,  k,          v, seq_lens, nullptr, out, mu_v, stats, B,
                            H_q, H_kv, H_q / H_kv, d, T,        S_max,   scale};
    return hip_status(parallax::launch_prefill(a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

size_t parallax_prefill_backward_workspace_size(int B, int H_q, int T, int d) {
  return bwd_workspace_bytes(B, H_q, T, d);
}

parallax_status_t parallax_prefill_backward(
    const void* q, const void* rho, const void* k, const void* v, const int32_t* seq_lens,
    const float* out, const float* mu_v, const float* stats, const float* dout, float* dq,
    float* drho, float* dk, float* dv, int B, int H_q, int H_kv, int d, int T, int S_max,
    float scale, parallax_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!q || !rho || !k || !v || !seq_lens || !out || !mu_v || !stats || !dout || !dq || !drho ||
        !dk || !dv || !workspace)
      return PARALLAX_ERR_NULL_POINTER;
    const parallax_status_t st = check_prefill_shape(B, H_q, H_kv, d, T, S_max, scale, dtype);
    if (st != PARALLAX_OK) return st;
    if (!aligned16(q) || !aligned16(rho) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(mu_v) || !aligned16(stats) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(drho) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
      return PARALLAX_ERR_MISALIGNED;
    if (workspace_bytes < bwd_workspace_bytes(B, H_q, T, d)) return PARALLAX_ERR_WORKSPACE;
    const size_t rows = (size_t)B * H_q * T;
    char* ws = static_cast<char*>(workspace);
    parallax::BwdArgs a;
    a.q = q;
    a.rho = rho;
    a.k = k;
    a.v = v;
    a.seq_lens = seq_lens;
    a.out = out;
    a.mu = mu_v;
    a.stats = reinterpret_cast<const float4*>(stats);
    a.dout = dout;
    a.dq = dq;
    a.drho = drho;
    a.dk = dk;
    a.dv = dv;
    a.dhi = reinterpret_cast<__bf16*>(ws);
    a.dlo = reinterpret_cast<__bf16*>(ws + rows * d * 2);
    a.gd = reinterpret_cast<float2*>(ws + 2 * rows * d * 2);
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = H_q / H_kv;
    a.d = d;
    a.T = T;
    a.S_max = S_max;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    return hip_status(parallax::launch_prefill_backward(a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

}  // extern "C"

extern "C" {

parallax_status_t parallax_qkvr_projection(const void* x, const void* w, void* q, void* rho,
                                           void* k_cache, void* v_cache,
                                           const int32_t* past_lens, int B, int T, int d_model,
                                           int H_q, int H_kv, int d, int S_max, void* stream) {
  try {
    if (!x || !w || !q || !rho || !k_cache || !v_cache) return PARALLAX_ERR_NULL_POINTER;
    if (B <= 0 || T <= 0 || d_model <= 0 || H_q <= 0 || H_kv <= 0 || d <= 0 || S_max <= 0 ||
        T > S_max || d_model % 64 != 0)
      return PARALLAX_ERR_BAD_SHAPE;
    if (d != 64 && d != 128) return PARALLAX_ERR_UNSUPPORTED;
    const long long N = (2LL * H_q + 2LL * H_kv) * d;
    // 32-bit buffer offsets within a 256-row tile; grid y = token tiles of 256
    if ((long long)B * T >= (1LL << 31) / 2 || 256LL * d_model * 2 >= (1LL << 31) ||
        N >= (1LL << 31) / 2 || ((long long)B * T + 255) / 256 > 65535)
      return PARALLAX_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(q) || !aligned16(rho) || !aligned16(k_cache) ||
        !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(past_lens) & 3u))
      return PARALLAX_ERR_MISALIGNED;
    parallax::ProjArgs a{x, w, q, k_cache, v_cache, rho, past_lens, B, T, d_model, H_q, H_kv, d,
                         S_max};
    return hip_status(parallax::launch_projection(a, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

}  // extern "C"

extern "C" {

parallax_status_t parallax_read_probe(const void* a, const void* b, size_t bytes_each,
                                      uint32_t* sink, int sink_words, void* stream) {
  try {
    if (!a || !b || !sink) return PARALLAX_ERR_NULL_POINTER;
    if (bytes_each == 0 || bytes_each % 16 != 0 || sink_words <= 0) return PARALLAX_ERR_BAD_SHAPE;
    if (!aligned16(a) || !aligned16(b) || (reinterpret_cast<uintptr_t>(sink) & 3u))
      return PARALLAX_ERR_MISALIGNED;
    const int cus = cu_count();
    if (cus <= 0) return PARALLAX_ERR_HIP;
    return hip_status(parallax::launch_read_probe(a, b, bytes_each, sink, (unsigned)sink_words,
                                                  2 * cus, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return PARALLAX_ERR_HIP;
  }
}

}  // extern "C"
