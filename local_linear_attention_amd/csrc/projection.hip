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
// Tiling. A workgroup of 4 waves computes 256 output features x 256 tokens;
// each wave 128 features x 128 tokens as 8 x 8 tiles of
// v_mfma_f32_16x16x32_bf16 with the features as the MFMA rows: 256
// accumulator registers, held in the accumulation registers at one wave per
// SIMD. The operand bytes a wave reads from LDS grow with its tile's rows
// plus columns while its MFMA work grows with their product, so the square
// 128 x 128 wave tile reads a third fewer LDS bytes per MFMA than two waves
// of 128 x 64 per SIMD (whose operand reads and staging writes kept the LDS
// as busy as the matrix pipe). K (d_model) advances 64 at a time through
// double-buffered LDS (chunks XOR-swizzled per row against bank conflicts).
// With one wave per SIMD nothing else hides a wave's LDS and global latency,
// so the wave pipelines its own: between the rows of one k-step's MFMAs it
// reads the next k-step's operands, and the next stage's first operands are
// read under the current stage's last MFMAs (one barrier per stage, between
// its two k-steps). On gfx950 every memory instruction a wave issues holds
// up its own MFMAs, so when d_model is a multiple of 128 the stages are
// loaded straight from global memory into LDS (buffer loads with the LDS
// flag, between the second k-step's MFMAs): no staging registers and no LDS
// store instructions (7% faster). Otherwise each stage goes through
// registers, stored into the other buffer between the first k-step's MFMAs.
// Loads past x's or W's rows come back as zeros (range-checked buffer loads).
//
// Epilogue. Each wave writes its tile to LDS token-major, then every token's
// 128 features (consecutive dims of one or two heads) leave as 16-byte stores,
// a contiguous 256-byte row segment per token.

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kWF = 128;                 // features per wave
constexpr int kWX = 128;                 // tokens per wave
constexpr int kNWF = 2;                  // waves along features
constexpr int kNWX = 2;                  // waves along tokens
constexpr int kThreads = 64 * kNWF * kNWX;
constexpr int kTileF = kWF * kNWF;       // 256 features per workgroup
constexpr int kTileX = kWX * kNWX;       // 256 tokens per workgroup
constexpr int kK = 64;                   // d_model per stage
constexpr int kStr = kK * 2;             // LDS row stride (bytes, unpadded)
// Byte offset of 16-byte chunk ch (0..7) of staged row r: the chunks of each
// row are permuted by an XOR with (r & 7) ^ ((r >> 3) & 1), so the operand
// reads (16 consecutive rows, one chunk) and the staging writes (whole rows)
// both spread over distinct banks.
__device__ __forceinline__ int swz(int r, int ch) { return (ch ^ ((r & 7) ^ ((r >> 3) & 1))) * 16; }
constexpr int kFI = kWF / 16;            // MFMA tiles per wave along features
constexpr int kXJ = kWX / 16;            // MFMA tiles per wave along tokens
constexpr int kPPW = kTileF * kK * 2 / 16 / kThreads;  // W pieces (16 bytes) per thread per stage
constexpr int kPPX = kTileX * kK * 2 / 16 / kThreads;  // x pieces per thread per stage
constexpr int kBuf = (kTileF + kTileX) * kStr;         // one LDS buffer: W tile then x tile
constexpr int kRowsPerLoad = 1024 / kStr;  // rows one wave-wide 16-byte load into LDS fills
constexpr int kLoads = (kTileF + kTileX) / kRowsPerLoad / (kThreads / 64);  // such loads per wave per stage
constexpr int kEStr = kWF * 2 + 16;      // epilogue: bytes per token row (16-byte aligned)
constexpr int kEHalf = kWX / 2;          // epilogue: tokens per pass
static_assert(kRowsPerLoad == 8 && kLoads == 16, "direct loads: 8 rows each, 16 per wave and stage");
static_assert(2 * kEHalf * kEStr <= kBuf, "two waves' epilogue halves must fit in one stage buffer");

// acc += a b (v_mfma_f32_16x16x32_bf16) with the accumulator bound to the
// accumulation registers. Left to itself the register allocator splits the
// 256 accumulator registers between the two register files and moves them
// every stage. Each accumulator is next used 64 MFMAs later (no dependency
// stall); the epilogue waits explicitly before reading them.
__device__ __forceinline__ void mfma_agpr(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// One workgroup per CU (its 4 waves, one per SIMD, may use the whole
// register file). DMA: stage loads go from global memory straight into LDS
// (needs d_model a multiple of 128: the stage loop runs in static pairs);
// otherwise through registers.
template <bool DMA>
__global__ __launch_bounds__(kThreads, 1) void proj_kernel(ProjArgs a) {
  // The two stage buffers are separate objects, so the compiler can tell a
  // read of one from a load still landing in the other.
  __shared__ __attribute__((aligned(16))) char lds0[kBuf];
  __shared__ __attribute__((aligned(16))) char lds1[kBuf];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int wf = wave / kNWX;  // feature half of the tile
  const int wx = wave % kNWX;  // token half of the tile
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
  // the next row (in range, unused) or past the last row (zeros). One
  // per-lane offset serves every piece: the row step 32 i and the stage
  // offset go in the scalar offset operand.
  const uint32_t voff = (uint32_t)(tid / 8) * KB + (tid % 8) * 16;
  const uint32_t loff = (uint32_t)(tid / 8) * kStr + swz(tid / 8, tid % 8);
  i32x4 sw[kPPW], sx[kPPX];
  auto load_piece = [&](int kt, int i) {
    const int soff = __builtin_amdgcn_readfirstlane(kt * kK * 2 + i * (kThreads / 8) * KB);
    sw[i] = __builtin_amdgcn_raw_buffer_load_b128(wrs, voff, soff, 0);
    sx[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, voff, soff, 0);
  };
  auto store_piece = [&](int buf, int i) {
    char* base = (buf ? lds1 : lds0) + loff + i * (kThreads / 8) * kStr;
    *reinterpret_cast<i32x4*>(base) = sw[i];
    *reinterpret_cast<i32x4*>(base + kTileF * kStr) = sx[i];
  };
  static_assert(kPPW == kPPX && kPPW == kFI, "one W and one x piece per feature row of MFMAs");

  f32x4 acc[kFI][kXJ];
#pragma unroll
  for (int i = 0; i < kFI; ++i)
#pragma unroll
    for (int j = 0; j < kXJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A operand of feature tile t in lane (g, c): feature row 16 t + c,
  // d_model 32 ks + 8 g .. + 7 of the stage; B operand of token tile t
  // likewise with token rows.
  auto rd_a = [&](const char* buf, int ks, int t) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(
        buf + (kWF * wf + 16 * t + c) * kStr + swz(c, g + 4 * ks)));
  };
  auto rd_b = [&](const char* buf, int ks, int t) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(
        buf + (kTileF + kWX * wx + 16 * t + c) * kStr + swz(c, g + 4 * ks)));
  };
  auto mfma_rows = [&](int i0, int i1, const bf16x8 (&af)[kFI], const bf16x8 (&bx)[kXJ]) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < kXJ; ++j) mfma_agpr(acc[i][j], af[i], bx[j]);
  };

  // Software pipeline, one barrier per stage. On entry to stage kt its
  // first k-step's operands (a0, b0) are in registers. Each feature row of
  // the first k-step's MFMAs is followed by two reads of the second k-step's
  // operands (and, staging through registers, the store of one W and one x
  // piece of stage kt + 1 into the other buffer and the loads of those pieces
  // of stage kt + 2). The barrier then publishes stage kt + 1; its first
  // operands are read while the second k-step's MFMAs run (and, loading
  // straight into LDS, stage kt + 2 is loaded between them into the buffer
  // just left). Loads past the last stage move zeros or unused data (or
  // repeat the last stage) and are never contracted.
  bf16x8 a0[kFI], b0[kXJ], a1[kFI], b1[kXJ];
  auto first_operands = [&](const char* buf) {
#pragma unroll
    for (int t = 0; t < kFI; ++t) a0[t] = rd_a(buf, 0, t);
#pragma unroll
    for (int t = 0; t < kXJ; ++t) b0[t] = rd_b(buf, 0, t);
  };
  const int nk = a.d_model / kK;
  // Direct loads: one wave-wide 16-byte load fills 1 KiB of LDS in lane
  // order, i.e. rows r0 .. r0 + 7 of a stage with lane L at row r0 + L / 8,
  // physical chunk L % 8; the lane fetches the logical chunk the swizzle
  // puts there. Wave w issues the loads of row blocks w, w + 4, .. (half in
  // W, half in x), so r0 / 8 has the parity of w and one lane offset serves
  // all of them.
  const int lrow = lane / 8;
  const uint32_t dvoff = (uint32_t)lrow * KB + 16 * ((lane % 8) ^ lrow ^ (wave & 1));
  auto direct_loads = [&](int kt, char* buf, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const bool isx = i >= kLoads / 2;
      const int r0 = kRowsPerLoad * (wave + (kThreads / 64) * (isx ? i - kLoads / 2 : i));
      const int soff = __builtin_amdgcn_readfirstlane(r0 * KB + kt * kK * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          isx ? xrs : wrs,
          (__attribute__((address_space(3))) void*)(buf + (isx ? kTileF * kStr : 0) + r0 * kStr), 16,
          dvoff, soff, 0, 0);
    }
  };
  if constexpr (DMA) {
    auto stage = [&](int kt, char* cur, char* nxt) {
#pragma unroll
      for (int i = 0; i < kFI; ++i) {
        mfma_rows(i, i + 1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        if (i < kFI / 2) {
          a1[2 * i] = rd_a(cur, 1, 2 * i);
          a1[2 * i + 1] = rd_a(cur, 1, 2 * i + 1);
        } else {
          b1[2 * i - kFI] = rd_b(cur, 1, 2 * i - kFI);
          b1[2 * i - kFI + 1] = rd_b(cur, 1, 2 * i - kFI + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();  // its fence waits for this wave's loads of stage kt + 1
      first_operands(nxt);  // past the last stage: unused
      __builtin_amdgcn_sched_barrier(0);
      const int kl = min(kt + 2, nk - 1);
#pragma unroll
      for (int i = 0; i < kFI; ++i) {
        direct_loads(kl, cur, 2 * i, 2 * i + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(i, i + 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    direct_loads(0, lds0, 0, kLoads);
    __syncthreads();
    first_operands(lds0);
    direct_loads(min(1, nk - 1), lds1, 0, kLoads);
    // A loop that may run zero times made the compiler zero the 256
    // accumulators twice (before and after its trip-count test).
    int kt = 0;
    do {  // nk is even and at least 2
      stage(kt, lds0, lds1);
      stage(kt + 1, lds1, lds0);
      kt += 2;
    } while (kt < nk);
    __syncthreads();  // no load still lands in a buffer the epilogue reuses
  } else {
    auto stage = [&](int kt, int buf) {
      const char* cur = buf ? lds1 : lds0;
#pragma unroll
      for (int i = 0; i < kFI; ++i) {
        mfma_rows(i, i + 1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        if (i < kFI / 2) {
          a1[2 * i] = rd_a(cur, 1, 2 * i);
          a1[2 * i + 1] = rd_a(cur, 1, 2 * i + 1);
        } else {
          b1[2 * i - kFI] = rd_b(cur, 1, 2 * i - kFI);
          b1[2 * i - kFI + 1] = rd_b(cur, 1, 2 * i - kFI + 1);
        }
        store_piece(buf ^ 1, i);
        load_piece(kt + 2, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      first_operands(buf ? lds0 : lds1);  // past the last stage: unused
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows(0, kFI, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int i = 0; i < kPPW; ++i) load_piece(0, i);
#pragma unroll
    for (int i = 0; i < kPPW; ++i) store_piece(0, i);
#pragma unroll
    for (int i = 0; i < kPPW; ++i) load_piece(1, i);
    __syncthreads();
    first_operands(lds0);
    int kt = 0;
    do {  // nk is at least 1
      stage(kt, kt & 1);
    } while (++kt < nk);
  }
  // the last MFMAs' results are read below: wait out their latency
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");

  // Epilogue: accumulator element e of lane (g, c) in tile (i, j) is feature
  // 16 i + 4 g + e, token 16 j + c of the wave. In two passes of 64 tokens it
  // goes to a token-major bf16 tile in LDS (waves 0 and 1 in one stage
  // buffer, waves 2 and 3 in the other); each token's 128 features are then
  // read back as 16 chunks of 8 and stored. After the last barrier the stage
  // buffers only see reads of operands that are never used and no load
  // lands in them, so each wave may overwrite its part (the parts are
  // disjoint) without another barrier.
  char* ep = ((wave >> 1) ? lds1 : lds0) + (wave & 1) * (kEHalf * kEStr);
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
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < kFI; ++i)
#pragma unroll
      for (int j = 0; j < kXJ / 2; ++j) {
        const f32x4 v = acc[i][j + half * (kXJ / 2)];
        const uint2 val = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        *reinterpret_cast<uint2*>(ep + (16 * j + c) * kEStr + (16 * i + 4 * g) * 2) = val;
      }
#pragma unroll 4
    for (int p = 0; p < kEHalf / kRPI; ++p) {
      const int r = kRPI * p + lane / kCH;
      const int m = X0 + kWX * wx + kEHalf * half + r;
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
}

}  // namespace

hipError_t launch_projection(const ProjArgs& a, hipStream_t st) {
  const int N = (2 * a.H_q + 2 * a.H_kv) * a.d;
  const int M = a.B * a.T;
  dim3 grid((N + kTileF - 1) / kTileF, (M + kTileX - 1) / kTileX);
  if (a.d_model % (2 * kK) == 0)
    hipLaunchKernelGGL(proj_kernel<true>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(proj_kernel<false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace parallax
