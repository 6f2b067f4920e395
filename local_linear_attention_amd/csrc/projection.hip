// Fused q, k, v, rho projection on CDNA4 (gfx950).
//
// Parallax learns its probe as a projection of the layer input, like the
// query (blog "Parallax: Breaking the Boundary Bias with Parameterized Local
// Linear Attention", "The Core Insight: Covariance Correction" and
// "Architecture-Optimizer Codesign", the W_R projection; paper page
// "Parallax: Parameterized Local Linear Attention for Language Modeling",
// "Abstract": a second projection of the input, used like a query). One GEMM produces all four
// projections of x, written in bf16 (round to nearest even) straight into the
// layouts the attention kernels read:
//
//   [q | k | v | rho] = x W^T,  W = [W_Q; W_K; W_V; W_R]  ((2 H_q + 2 H_kv) d rows, d_model cols)
//   q, rho -> [B, H_q, T, d];  k, v -> rows past_b + t of the cache [B, H_kv, S_max, d]
//
// Tiling. A workgroup of 8 waves computes 256 output features x 256 tokens;
// each wave 128 features x 64 tokens as 8 x 4 tiles of
// v_mfma_f32_16x16x32_bf16 with the features as the MFMA rows (128
// accumulator registers; two waves per SIMD). The larger wave tile halves
// the LDS operand reads per MFMA against 64 x 64 wave tiles. K (d_model)
// advances 64 at a time through double-buffered LDS (rows padded by 16 bytes
// so the 16-row operand reads hit distinct banks), with two register stages
// so each global load has two stages of contraction to land. Within a k-step
// the operand reads of half the feature tiles are issued before their MFMAs
// (order pinned by scheduling barriers). Loads past x's or W's rows come back
// as zeros (range-checked buffer loads).
//
// Epilogue. Each wave writes its tile to LDS token-major, then every token's
// 128 features (consecutive dims of one or two heads) leave as 16-byte stores,
// a contiguous 256-byte row segment per token.

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kWF = 128;                 // features per wave
constexpr int kWX = 64;                  // tokens per wave
constexpr int kNWF = 2;                  // waves along features
constexpr int kNWX = 4;                  // waves along tokens
constexpr int kThreads = 64 * kNWF * kNWX;
constexpr int kTileF = kWF * kNWF;       // 256 features per workgroup
constexpr int kTileX = kWX * kNWX;       // 256 tokens per workgroup
constexpr int kK = 64;                   // d_model per stage
constexpr int kStr = kK * 2 + 16;        // LDS row stride (bytes)
constexpr int kFI = kWF / 16;            // MFMA tiles per wave along features
constexpr int kXJ = kWX / 16;            // MFMA tiles per wave along tokens
constexpr int kPPW = kTileF * kK * 2 / 16 / kThreads;  // W pieces (16 bytes) per thread per stage
constexpr int kPPX = kTileX * kK * 2 / 16 / kThreads;  // x pieces per thread per stage
constexpr int kBuf = (kTileF + kTileX) * kStr;         // one LDS buffer: W tile then x tile
constexpr int kEStr = kWF * 2 + 16;      // epilogue: bytes per token row (16-byte aligned)
static_assert(kNWF * kNWX * kWX * kEStr <= 2 * kBuf, "epilogue tiles must fit in the stage buffers");

__global__ __launch_bounds__(kThreads) void proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kBuf];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int wf = wave / kNWX;  // feature half of the tile
  const int wx = wave % kNWX;  // token quarter of the tile
  // Tile order. Workgroups are dealt to the 8 XCDs in linear order: remap so
  // each XCD takes a contiguous range, and walk that range in groups of 8 x 8
  // (token, feature) tiles, so the workgroups an XCD runs at once share 8
  // token tiles of x and 8 feature tiles of W in its L2 (when the tile counts
  // are multiples of 8).
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

  // Byte sizes of the workgroup's W and x rows. The compiler clamps them on
  // the vector ALU; readfirstlane returns them to scalar registers, or every
  // buffer load would be wrapped in a loop over the distinct descriptors.
  const uint32_t wbytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(kTileF, N - F0)) * KB);
  const uint32_t xbytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(kTileX, M - X0)) * KB);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(static_cast<const __bf16*>(a.w) + (size_t)F0 * a.d_model, wbytes);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(static_cast<const __bf16*>(a.x) + (size_t)X0 * a.d_model, xbytes);

  // Thread tid's pieces: rows (tid + kThreads i) / 8, 16-byte column
  // (tid + kThreads i) % 8 of the stage. Past d_model the offsets run into
  // the next row (in range, unused) or past the last row (zeros).
  // The stage offset kt * 128 bytes goes in the scalar offset operand.
  auto load = [&](int kt, i32x4 (&sw)[kPPW], i32x4 (&sx)[kPPX]) {
    const int soff = __builtin_amdgcn_readfirstlane(kt * kK * 2);
#pragma unroll
    for (int i = 0; i < kPPW; ++i) {
      const int idx = tid + kThreads * i;
      sw[i] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (uint32_t)(idx / 8) * KB + (idx % 8) * 16, soff, 0);
    }
#pragma unroll
    for (int i = 0; i < kPPX; ++i) {
      const int idx = tid + kThreads * i;
      sx[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (uint32_t)(idx / 8) * KB + (idx % 8) * 16, soff, 0);
    }
  };
  auto store = [&](int buf, const i32x4 (&sw)[kPPW], const i32x4 (&sx)[kPPX]) {
    char* base = lds + buf * kBuf;
#pragma unroll
    for (int i = 0; i < kPPW; ++i) {
      const int idx = tid + kThreads * i;
      *reinterpret_cast<i32x4*>(base + (idx / 8) * kStr + (idx % 8) * 16) = sw[i];
    }
#pragma unroll
    for (int i = 0; i < kPPX; ++i) {
      const int idx = tid + kThreads * i;
      *reinterpret_cast<i32x4*>(base + (kTileF + idx / 8) * kStr + (idx % 8) * 16) = sx[i];
    }
  };

  f32x4 acc[kFI][kXJ];
#pragma unroll
  for (int i = 0; i < kFI; ++i)
#pragma unroll
    for (int j = 0; j < kXJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One stage from LDS buffer buf. A operand of feature tile t in lane
  // (g, c): feature row 16 t + c, d_model 32 ks + 8 g .. + 7; B operand of
  // token tile t likewise with token rows.
  auto compute = [&](int buf) {
    const char* wb = lds + buf * kBuf + (kWF * wf + c) * kStr + 16 * g;
    const char* xb = lds + buf * kBuf + (kTileF + kWX * wx + c) * kStr + 16 * g;
#pragma unroll
    for (int ks = 0; ks < kK / 32; ++ks) {
      bf16x8 bx[kXJ];
#pragma unroll
      for (int t = 0; t < kXJ; ++t)
        bx[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(xb + 16 * t * kStr + 64 * ks));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 af[kFI / 2];
#pragma unroll
        for (int t = 0; t < kFI / 2; ++t)
          af[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(
                      wb + 16 * (t + hf * kFI / 2) * kStr + 64 * ks));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kFI / 2; ++i)
#pragma unroll
          for (int j = 0; j < kXJ; ++j)
            acc[i + hf * kFI / 2][j] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bx[j], acc[i + hf * kFI / 2][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Stage kt is contracted from buffer kt % 2 while stage kt + 1 goes from
  // registers into the other buffer and stage kt + 3 is loaded into the
  // registers just freed. The loop is unrolled by two so that the register
  // stage of each step is static; stores and loads past the last stage move
  // zeros or unused data and are never contracted.
  i32x4 sw[2][kPPW], sx[2][kPPX];
  const int nk = a.d_model / kK;
  load(0, sw[0], sx[0]);
  load(1, sw[1], sx[1]);
  store(0, sw[0], sx[0]);
  load(2, sw[0], sx[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    compute(0);
    store(1, sw[1], sx[1]);
    load(kt + 3, sw[1], sx[1]);
    __syncthreads();
    if (kt + 1 < nk) compute(1);
    store(0, sw[0], sx[0]);
    load(kt + 4, sw[0], sx[0]);
    __syncthreads();
  }

  // Epilogue: accumulator element e of lane (g, c) in tile (i, j) is feature
  // 16 i + 4 g + e, token 16 j + c of the wave. It goes to a token-major bf16
  // tile in LDS (the stage buffers are free after the last barrier); each
  // token's 128 features are then read back as 16 chunks of 8 and stored.
  char* ep = lds + wave * (kWX * kEStr);
#pragma unroll
  for (int i = 0; i < kFI; ++i)
#pragma unroll
    for (int j = 0; j < kXJ; ++j) {
      const uint2 val = {pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
      *reinterpret_cast<uint2*>(ep + (16 * j + c) * kEStr + (16 * i + 4 * g) * 2) = val;
    }
  constexpr int kCH = kWF / 8;   // 16-byte chunks per token row
  constexpr int kRPI = 64 / kCH;  // token rows per pass of the wave
  const int ch = lane % kCH;
  const int f = F0 + kWF * wf + 8 * ch;  // first of the chunk's 8 features (never straddles a head: 8 | d)
  const int Fq = a.H_q * a.d, Fk = a.H_kv * a.d;
  int seg = 0, fr = f;  // 0 q, 1 k, 2 v, 3 rho; fr = feature within the segment
  if (fr >= Fq) { fr -= Fq; seg = 1;
    if (fr >= Fk) { fr -= Fk; seg = 2;
      if (fr >= Fk) { fr -= Fk; seg = 3; } } }
  const int h = fr / a.d;
  const int dim = fr % a.d;
#pragma unroll
  for (int p = 0; p < kWX / kRPI; ++p) {
    const int r = kRPI * p + lane / kCH;
    const int m = X0 + kWX * wx + r;
    if (m >= M || f >= N) continue;
    const int b = m / a.T;
    const int t = m % a.T;
    const i32x4 val = *reinterpret_cast<const i32x4*>(ep + r * kEStr + 16 * ch);
    __bf16* dst;
    if (seg == 0 || seg == 3) {
      dst = static_cast<__bf16*>(seg == 0 ? a.q : a.rho) + (((size_t)b * a.H_q + h) * a.T + t) * a.d + dim;
    } else {
      const int pos = (a.past_lens ? min(max(a.past_lens[b], 0), a.S_max) : 0) + t;
      if (pos >= a.S_max) continue;
      dst = static_cast<__bf16*>(seg == 1 ? a.k : a.v) + (((size_t)b * a.H_kv + h) * a.S_max + pos) * a.d + dim;
    }
    *reinterpret_cast<i32x4*>(dst) = val;
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
