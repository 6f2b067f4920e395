// Fused q, k, v, rho projection on CDNA4 (gfx950).
//
// Parallax learns its probe as a projection of the layer input, like the
// query (blog "Parallax: Breaking the Boundary Bias with Parameterized Local
// Linear Attention", "The Core Insight: Covariance Correction" and
// "Architecture-Optimizer Codesign", the W_R projection; paper page
// "Parallax: Parameterized Local Linear Attention for Language Modeling",
// "Abstract": an extra query-like projector). One GEMM produces all four
// projections of x, written in bf16 (round to nearest even) straight into the
// layouts the attention kernels read:
//
//   [q | k | v | rho] = x W^T,  W = [W_Q; W_K; W_V; W_R]  ((2 H_q + 2 H_kv) d rows, d_model cols)
//   q, rho -> [B, H_q, T, d];  k, v -> rows past_b + t of the cache [B, H_kv, S_max, d]
//
// Tiling. A workgroup of 4 waves computes 128 output features x 128 tokens;
// each wave 64 x 64 as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16 with the
// features as the MFMA rows, so each lane ends with 4 consecutive features
// of one token: one 8-byte store per tile into the head-major layout. K
// (d_model) advances 64 at a time through double-buffered LDS (rows padded by
// 16 bytes so the 16-row operand reads hit distinct banks), one register stage
// in flight. Loads past x's rows come back as zeros (range-checked buffer
// loads).

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kThreads = 256;
constexpr int kTileF = 128;  // features per workgroup
constexpr int kTileX = 128;  // tokens per workgroup
constexpr int kK = 64;       // d_model per stage
constexpr int kStr = kK * 2 + 16;  // LDS row stride (bytes)
constexpr int kPieces = 128 * kK * 2 / 16;  // 16-byte pieces per operand tile
constexpr int kPPT = 2 * kPieces / kThreads;  // pieces per thread per stage

__global__ __launch_bounds__(kThreads) void proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][128 * kStr];  // [buffer][W, x]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int wf = wave >> 1;  // feature half of the tile
  const int wx = wave & 1;   // token half of the tile
  // Tile order. Workgroups are dealt to the 8 XCDs in linear order: remap so
  // each XCD takes a contiguous range, and walk that range in groups of 8 x 8
  // (token, feature) tiles, so the ~64 workgroups an XCD runs at once share
  // 8 token tiles of x and 8 feature tiles of W in its L2 instead of all
  // feature tiles of W (when the tile counts are multiples of 8).
  int ft = blockIdx.x, xt = blockIdx.y;
  {
    const unsigned nf = gridDim.x, nx = gridDim.y, total = nf * nx;  // < 2^31: host-checked
    if (nf % 8u == 0u && nx % 8u == 0u) {
      const unsigned lin = blockIdx.x + nf * blockIdx.y;
      const unsigned L = (lin % 8u) * (total / 8u) + lin / 8u;
      const unsigned st = L / 64u, w = L % 64u;  // 8 x 8 super-tile, position in it
      const unsigned sf = nf / 8u;
      ft = (int)(8u * (st % sf) + w % 8u);
      xt = (int)(8u * (st / sf) + w / 8u);
    }
  }
  const int F0 = ft * kTileF;
  const int X0 = xt * kTileX;
  const int M = a.B * a.T;
  const int N = (2 * a.H_q + 2 * a.H_kv) * a.d;
  const int KB = a.d_model * 2;  // bytes per row of x and W

  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(static_cast<const __bf16*>(a.w) + (size_t)F0 * a.d_model, (uint32_t)min(kTileF, N - F0) * KB);
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(static_cast<const __bf16*>(a.x) + (size_t)X0 * a.d_model, (uint32_t)max(0, min(kTileX, M - X0)) * KB);

  i32x4 st[kPPT];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kPPT; ++i) {
      const int which = i < kPPT / 2 ? 0 : 1;  // W pieces, then x pieces
      const int idx = tid + kThreads * (i % (kPPT / 2));
      const int r = idx / (kK * 2 / 16);
      const int c16 = idx % (kK * 2 / 16);
      const uint32_t off = (uint32_t)r * KB + (uint32_t)kt * kK * 2 + c16 * 16;
      st[i] = __builtin_amdgcn_raw_buffer_load_b128(which ? xrs : wrs, off, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPPT; ++i) {
      const int which = i < kPPT / 2 ? 0 : 1;
      const int idx = tid + kThreads * (i % (kPPT / 2));
      const int r = idx / (kK * 2 / 16);
      const int c16 = idx % (kK * 2 / 16);
      *reinterpret_cast<i32x4*>(&lds[buf][which][r * kStr + c16 * 16]) = st[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.d_model / kK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    load(kt + 1);  // past d_model: offsets beyond each row, unused
#pragma unroll
    for (int ks = 0; ks < kK / 32; ++ks) {
      bf16x8 af[4], bx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(
                    &lds[buf][0][(64 * wf + 16 * t + c) * kStr + 64 * ks + 16 * g]));
        bx[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(
                    &lds[buf][1][(64 * wx + 16 * t + c) * kStr + 64 * ks + 16 * g]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bx[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // lane (g, c) of tile (i, j): features F0 + 64 wf + 16 i + 4 g + (0..3), token X0 + 64 wx + 16 j + c
  const int Fq = a.H_q * a.d, Fk = a.H_kv * a.d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = F0 + 64 * wf + 16 * i + 4 * g;
    if (f >= N) continue;
    int seg = 0, fr = f;  // 0 q, 1 k, 2 v, 3 rho; fr = feature within the segment
    if (fr >= Fq) { fr -= Fq; seg = 1;
      if (fr >= Fk) { fr -= Fk; seg = 2;
        if (fr >= Fk) { fr -= Fk; seg = 3; } } }
    const int h = fr / a.d;
    const int dim = fr % a.d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = X0 + 64 * wx + 16 * j + c;
      if (m >= M) continue;
      const int b = m / a.T;
      const int t = m % a.T;
      const uint2 val = {pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
      __bf16* dst;
      if (seg == 0 || seg == 3) {
        dst = static_cast<__bf16*>(seg == 0 ? a.q : a.rho) + (((size_t)b * a.H_q + h) * a.T + t) * a.d + dim;
      } else {
        const int pos = (a.past_lens ? min(max(a.past_lens[b], 0), a.S_max) : 0) + t;
        if (pos >= a.S_max) continue;
        dst = static_cast<__bf16*>(seg == 1 ? a.k : a.v) + (((size_t)b * a.H_kv + h) * a.S_max + pos) * a.d + dim;
      }
      *reinterpret_cast<uint2*>(dst) = val;
    }
  }
}

}  // namespace

hipError_t launch_projection(const ProjArgs& a, hipStream_t st) {
  const int N = (2 * a.H_q + 2 * a.H_kv) * a.d;
  const int M = a.B * a.T;
  dim3 grid((N + kTileF - 1) / kTileF, (M + kTileX - 1) / kTileX);
  hipLaunchKernelGGL(proj_kernel, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace parallax
