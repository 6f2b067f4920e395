// Host-side check of the C ABI (api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU. Built by
// tests/test_abi_host_sanitized.py from api.cpp alone: the kernel launchers
// and the two device queries api.cpp makes are replaced here, so every
// argument check, the split plan and the marshalling of launch arguments run
// as in the library, and each would-be launch is recorded instead of run.
//
// Checked: argument errors return their status and launch nothing; valid
// calls launch exactly once with the planned split count and chunk and the
// caller's workspace; the plan's invariants hold over a grid of shapes that
// includes the extremes of every int argument; no size computation
// overflows (UBSan traps on signed overflow; unsigned sizes are compared
// with 128-bit arithmetic here). Exit status 0 when every check passes.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "kernels.h"
#include "parallax.h"

// ---- replacements for what api.cpp needs from the HIP runtime and kernels
static int g_launches = 0;
static parallax::DecodeArgs g_dec;

extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}

namespace parallax {
hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t) {
  ++g_launches;
  g_dec = a;
  return hipSuccess;
}
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t) {
  ++g_launches;
  g_dec = a;
  return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_backward(const BwdArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_projection(const ProjArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_read_probe(const void*, const void*, size_t, uint32_t*, unsigned, int,
                             hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace parallax

// ---- checks
static int g_failures = 0;

#define CHECK(cond, ...)                       \
  do {                                         \
    if (!(cond)) {                             \
      ++g_failures;                            \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                \
      std::printf("\n");                       \
    }                                          \
  } while (0)

// Fake device addresses: 16-byte aligned, never dereferenced on the host.
static void* P(uintptr_t i) { return reinterpret_cast<void*>(0x100000 + 0x1000 * i); }
static const int32_t* I(uintptr_t i) { return static_cast<const int32_t*>(P(i)); }
static float* F(uintptr_t i) { return static_cast<float*>(P(i)); }

typedef unsigned __int128 u128;

static void plan_grid() {
  const int Bs[] = {-1, 0, 1, 8, 64, 65535, 65536, INT_MAX};
  const int hs[][2] = {{1, 1}, {16, 8}, {64, 8}, {32, 8}, {6, 1}, {3, 2}, {INT_MAX, 1}, {0, 1}};
  const int ds[] = {0, 32, 64, 128, 256};
  const int Ss[] = {-1, 0, 1, 127, 128, 129, 4096, 131072, 8388543, INT_MAX - 128, INT_MAX - 127,
                    INT_MAX};
  const int reqs[] = {-1, 0, 1, 3, 32, 65535, 65536, INT_MAX};
  for (int B : Bs)
    for (auto& h : hs)
      for (int d : ds)
        for (int S : Ss)
          for (int r : reqs) {
            int ns = -7, chunk = -7;
            const parallax_status_t st = parallax_decode_plan(B, h[0], h[1], d, S, r, &ns, &chunk);
            if (st != PARALLAX_OK) continue;
            CHECK(ns >= 1 && chunk >= 128 && chunk % 128 == 0,
                  "plan(%d,%d,%d,%d,%d,%d): ns %d chunk %d", B, h[0], h[1], d, S, r, ns, chunk);
            CHECK((long long)ns * chunk >= S, "plan(%d,%d,%d,%d,%d,%d) covers %lld < %d keys", B,
                  h[0], h[1], d, S, r, (long long)ns * chunk, S);
            CHECK((long long)(ns - 1) * chunk < S, "plan(%d,%d,%d,%d,%d,%d): empty last split", B,
                  h[0], h[1], d, S, r);
            const size_t ws = parallax_decode_workspace_size(B, h[0], d, ns);
            if (ns > 1) {
              const u128 rec = (u128)B * (u128)h[0] * (u128)ns * (u128)(2 * d + 4) * 4u;
              // either the exact size, or 0 for a plan no call accepts
              CHECK(ws == 0 || (u128)ws >= rec, "workspace_size(%d,%d,%d,%d) = %zu wrapped", B,
                    h[0], d, ns, ws);
            } else {
              CHECK(ws == 0, "one-split plan needs no workspace");
            }
          }
}

static void decode_calls() {
  // valid gqa-decode shape: one launch with the plan's splits and the workspace
  int ns = 0, chunk = 0;
  CHECK(parallax_decode_plan(8, 16, 8, 128, 4096, 0, &ns, &chunk) == PARALLAX_OK, "plan");
  const size_t ws = parallax_decode_workspace_size(8, 16, 128, ns);
  g_launches = 0;
  parallax_status_t st = parallax_decode(P(1), P(2), P(3), P(4), I(5), F(6), 8, 16, 8, 128, 4096,
                                         1.0f, PARALLAX_BF16, 0, P(7), ws, nullptr);
  CHECK(st == PARALLAX_OK && g_launches == 1, "decode: status %d, %d launches", st, g_launches);
  CHECK(g_dec.num_splits == ns && g_dec.chunk == chunk && g_dec.ws == P(7) && g_dec.counters != nullptr,
        "decode launch arguments");
  CHECK(static_cast<char*>(g_dec.counters) + 8 * 16 * 4 <= static_cast<char*>(P(7)) + ws,
        "counters inside the workspace");

  struct Bad {
    int B, H_q, H_kv, d, S;
    float scale;
    int dtype, splits;
    size_t ws;
    parallax_status_t want;
  };
  const Bad bad[] = {
      {0, 16, 8, 128, 4096, 1.f, 0, 0, ws, PARALLAX_ERR_BAD_SHAPE},
      {8, 16, 7, 128, 4096, 1.f, 0, 0, ws, PARALLAX_ERR_BAD_SHAPE},
      {8, 16, 8, 96, 4096, 1.f, 0, 0, ws, PARALLAX_ERR_UNSUPPORTED},
      {8, 16, 8, 128, 4096, NAN, 0, 0, ws, PARALLAX_ERR_BAD_SHAPE},
      {8, 16, 8, 128, 4096, INFINITY, 0, 0, ws, PARALLAX_ERR_BAD_SHAPE},
      {8, 16, 8, 128, 4096, 1.f, 2, 0, ws, PARALLAX_ERR_UNSUPPORTED},
      {8, 16, 8, 128, 4096, 1.f, 0, -1, ws, PARALLAX_ERR_BAD_SHAPE},
      {8, 16, 8, 128, 4096, 1.f, 0, 0, ws - 1, PARALLAX_ERR_WORKSPACE},
      {65536, 16, 8, 128, 4096, 1.f, 0, 0, ws, PARALLAX_ERR_UNSUPPORTED},
      {8, 16, 8, 128, INT_MAX, 1.f, 0, 0, ws, PARALLAX_ERR_UNSUPPORTED},
      {8, 16, 8, 128, 4096, 1.f, 0, 65536, ws, PARALLAX_ERR_WORKSPACE},  // 32 chunks of 128
      {1, 1, 1, 64, 1 << 23, 1.f, 0, 65536, ws, PARALLAX_ERR_UNSUPPORTED},  // 65536 splits
  };
  for (const Bad& b : bad) {
    g_launches = 0;
    st = parallax_decode(P(1), P(2), P(3), P(4), I(5), F(6), b.B, b.H_q, b.H_kv, b.d, b.S, b.scale,
                         (parallax_dtype_t)b.dtype, b.splits, P(7), b.ws, nullptr);
    CHECK(st != PARALLAX_OK && g_launches == 0, "bad decode (B %d, d %d, S %d): status %d, %d launches",
          b.B, b.d, b.S, st, g_launches);
    CHECK(b.want == st, "bad decode (B %d, H %d/%d, d %d, S %d, splits %d): status %d, expected %d",
          b.B, b.H_q, b.H_kv, b.d, b.S, b.splits, st, b.want);
  }
  g_launches = 0;
  st = parallax_decode(P(1), P(2), P(3), P(4), I(5), F(6), 8, 16, 8, 128, 4096, 1.f, PARALLAX_BF16,
                       0, reinterpret_cast<char*>(P(7)) + 4, ws, nullptr);
  CHECK(st == PARALLAX_ERR_MISALIGNED && g_launches == 0, "misaligned workspace: %d", st);
  st = parallax_decode(nullptr, P(2), P(3), P(4), I(5), F(6), 8, 16, 8, 128, 4096, 1.f,
                       PARALLAX_BF16, 0, P(7), ws, nullptr);
  CHECK(st == PARALLAX_ERR_NULL_POINTER && g_launches == 0, "null q: %d", st);

  // huge head counts: either refused, or a workspace size that did not wrap
  for (int H : {1 << 20, 1 << 26, 1 << 30, INT_MAX}) {
    int n2 = 0, c2 = 0;
    if (parallax_decode_plan(65535, H, 1, 128, 1 << 20, 65535, &n2, &c2) != PARALLAX_OK) continue;
    const size_t w2 = parallax_decode_workspace_size(65535, H, 128, n2);
    const u128 rec = (u128)65535 * (u128)H * (u128)n2 * 260u * 4u;
    CHECK(w2 == 0 || (u128)w2 >= rec, "workspace_size(65535, %d, 128, %d) = %zu wrapped", H, n2, w2);
    g_launches = 0;
    st = parallax_decode(P(1), P(2), P(3), P(4), I(5), F(6), 65535, H, 1, 128, 1 << 20, 1.f,
                         PARALLAX_BF16, 65535, P(7), w2, nullptr);
    CHECK(st != PARALLAX_OK || (u128)w2 >= rec, "decode accepted a wrapped workspace (H_q %d)", H);
  }

  // multi-token decode: T > S_max and T overflowing H_q * T are refused
  g_launches = 0;
  st = parallax_decode_tokens(P(1), P(2), P(3), P(4), I(5), I(6), F(7), 8, 16, 8, 128, 4097, 4096,
                              1.f, PARALLAX_BF16, 0, P(8), 1 << 30, nullptr);
  CHECK(st == PARALLAX_ERR_BAD_SHAPE && g_launches == 0, "tokens T > S_max: %d", st);
  st = parallax_decode_tokens(P(1), P(2), P(3), P(4), I(5), I(6), F(7), 8, 1 << 20, 8, 128, 4096,
                              1 << 20, 1.f, PARALLAX_BF16, 0, P(8), 1 << 30, nullptr);
  CHECK(st != PARALLAX_OK && g_launches == 0, "tokens H_q * T overflow accepted: %d", st);
}

static void prefill_calls() {
  g_launches = 0;
  parallax_status_t st = parallax_prefill(P(1), P(2), P(3), P(4), I(5), F(6), 4, 16, 8, 128, 4096,
                                          4096, 1.f, PARALLAX_BF16, nullptr);
  CHECK(st == PARALLAX_OK && g_launches == 1, "prefill: %d, %d launches", st, g_launches);
  const int shapes[][6] = {
      // B, H_q, H_kv, d, T, S_max
      {4, 16, 8, 128, 4097, 4096}, {4, 16, 8, 128, 0, 4096}, {4, 16, 6, 128, 64, 64},
      {4, 16, 8, 80, 64, 64},      {INT_MAX, INT_MAX, 1, 128, INT_MAX, INT_MAX},
      {65536, 16, 8, 128, 64, 64}, {1, 1, 1, 128, 1 << 30, 1 << 30},
  };
  for (auto& s : shapes) {
    g_launches = 0;
    st = parallax_prefill(P(1), P(2), P(3), P(4), I(5), F(6), s[0], s[1], s[2], s[3], s[4], s[5],
                          1.f, PARALLAX_BF16, nullptr);
    CHECK(st != PARALLAX_OK && g_launches == 0, "prefill (%d,%d,%d,%d,%d,%d) accepted", s[0], s[1],
          s[2], s[3], s[4], s[5]);
    st = parallax_prefill_chunked(P(1), P(2), P(3), P(4), I(5), I(6), F(7), s[0], s[1], s[2], s[3],
                                  s[4], s[5], 1.f, PARALLAX_BF16, nullptr);
    CHECK(st != PARALLAX_OK && g_launches == 0, "chunked (%d,%d,%d,%d,%d,%d) accepted", s[0], s[1],
          s[2], s[3], s[4], s[5]);
  }
  // backward: workspace size and its check
  const size_t bws = parallax_prefill_backward_workspace_size(4, 16, 4096, 128);
  CHECK(bws > 0, "backward workspace size");
  CHECK(parallax_prefill_backward_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128) == 0 ||
            (u128)parallax_prefill_backward_workspace_size(INT_MAX, INT_MAX, INT_MAX, 128) >=
                (u128)INT_MAX * INT_MAX * INT_MAX,
        "backward workspace size wrapped");
}

static void projection_and_probe_calls() {
  g_launches = 0;
  parallax_status_t st = parallax_qkvr_projection(P(1), P(2), P(3), P(4), P(5), P(6), I(7), 4, 4096,
                                                  2048, 16, 8, 128, 4096, nullptr);
  CHECK(st == PARALLAX_OK && g_launches == 1, "projection: %d, %d launches", st, g_launches);
  const int shapes[][7] = {
      // B, T, d_model, H_q, H_kv, d, S_max
      {4, 4096, 2000, 16, 8, 128, 4096},          {4, 4097, 2048, 16, 8, 128, 4096},
      {INT_MAX, INT_MAX, 2048, 16, 8, 128, INT_MAX}, {1, 64, 2048, INT_MAX, INT_MAX, 128, 64},
      {1, 64, INT_MAX - 63, 16, 8, 128, 64},      {1, 64, 2048, 16, 8, 96, 64},
  };
  for (auto& s : shapes) {
    g_launches = 0;
    st = parallax_qkvr_projection(P(1), P(2), P(3), P(4), P(5), P(6), I(7), s[0], s[1], s[2], s[3],
                                  s[4], s[5], s[6], nullptr);
    CHECK(st != PARALLAX_OK && g_launches == 0, "projection (%d,%d,%d,%d,%d,%d,%d) accepted", s[0],
          s[1], s[2], s[3], s[4], s[5], s[6]);
  }
  g_launches = 0;
  st = parallax_read_probe(P(1), P(2), (size_t)1 << 30, reinterpret_cast<uint32_t*>(P(3)), 4096,
                           nullptr);
  CHECK(st == PARALLAX_OK && g_launches == 1, "read probe: %d", st);
  st = parallax_read_probe(P(1), P(2), 17, reinterpret_cast<uint32_t*>(P(3)), 4096, nullptr);
  CHECK(st == PARALLAX_ERR_BAD_SHAPE && g_launches == 1, "read probe of 17 bytes: %d", st);
}

int main() {
  plan_grid();
  decode_calls();
  prefill_calls();
  projection_and_probe_calls();
  std::printf("%s (%d failures)\n", g_failures ? "FAILED" : "ok", g_failures);
  return g_failures ? 1 : 0;
}
