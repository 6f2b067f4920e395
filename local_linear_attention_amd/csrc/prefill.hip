// Parallax causal prefill on CDNA4 (gfx950).
//
// Row t of sequence b, query head h, sees keys 0..t of KV head h / G (with a
// per-sequence past length p, the chunked form: row t sits at position p + t
// and sees keys 0..p + t of the cache, which already holds the chunk's keys)
// ("Parallax: Parameterized Local Linear Attention for Language Modeling",
// paper page, "Abstract": the extra projector rho is query-like, so it is per
// token here like q; blog "Parallax: Breaking the Boundary Bias with
// Parameterized Local Linear Attention", "The Core Insight: Covariance
// Correction", output equation):
//
//   out_t = mu_v - S_KV rho_t = (A (1 + Bs/l) - C) / l
//
// with, over keys j <= t, e_j = exp(s_tj - m), s_tj = scale q_t.k_j,
// r_tj = rho_t.k_j - c_t, l = sum e, A = sum e v_j, Bs = sum e r, C = sum e r v_j.
// Any per-row reference c_t cancels exactly (it shifts Bs by c l and C by
// c A); it keeps a large common offset of rho.k out of the accumulated
// products.
//
// Tiling. A workgroup of 8 waves owns 128 query rows of one (b, h); each wave
// owns 16 rows, so a wave needs about 195-202 registers and two waves share each
// SIMD (while one waits on LDS or on a dependency the other issues; on gfx950
// MFMA and VALU instructions of one SIMD never execute at the same time).
// Key blocks of 32 keys are staged two at a time in double-buffered LDS (rows
// padded against bank conflicts), shared by the 8 waves, and loaded one pair
// before use. Per wave and key block, v_mfma_f32_16x16x32_bf16 computes the
// transposed scores S^T = K Q^T and R^T = K rho^T for two 16-key tiles: lane
// (g = lane / 16, c = lane % 16) holds query row c for keys 16 T + 4 g + i
// (T = 0, 1; i = 0..3), which are exactly the 8 key slots that lane supplies
// as the A operand of the value MFMA, so no data moves between lanes; row
// statistics need two exchanges (lanes ^ 16, ^ 32). The value MFMA computes
// [e; e r] V. The V operand (key slots down, dims across) comes straight
// from the row-major V tile through the CDNA4 transposing LDS load
// (ds_read_b64_tr_b16), so no lane shuffles V in registers; output column c
// of N-tile j is dim 16 j + c. Softmax rescaling is lazy (only when a block's
// max exceeds the running reference by more than 2^8). Each workgroup handles
// a heavy (late) and a light (early) row block, so every workgroup carries
// the same causal work.
//
// Short chunks (at most 256 rows, e.g. a few new tokens after a long cache)
// would leave most of the chip idle with 128-row blocks paired per
// workgroup. They take 16-row (up to 32 rows), 32-row (up to 64) or 64-row
// blocks, one per workgroup, and split each row block's keys into NS
// contiguous ranges (4, 4 and 2): a step stages the next block of every
// range, each of the first NS TL waves (TL tiles of 16 rows per range)
// contracts its own range's block, any remaining waves only help stage, and
// at the end the ranges' (m, l, Bs, c, A, C) merge in LDS into the range-0
// waves. Each step's loads are issued two steps ahead.
//
// Weights of the value contraction. Inference (prefill, chunked prefill):
// e and e (r - c) are rounded once to fp16 and V is staged as fp16 (exact for
// bf16 values of magnitude 2^-14 .. 65504), two products per value tile.
// l and Bs sum the same rounded weights, so A / l is an exact weighted mean
// under weights perturbed by less than 2^-10 of themselves; the probe
// reference c follows the running weighted mean of r (moved on the first
// block and whenever a block's max jumps by more than 2^3), so the rounding
// of e (r - c) stays small next to the weights that dominate a row. Measured
// against the fp64 oracle: 3-6e-4 per row at the benchmark statistics, up to
// about 1.3e-3 with probes 20x stronger and a sharp softmax. Training
// forward (also writes mu_v and the row statistics the backward recomputes
// the weights from): e and e (r - c) as a bf16 high part plus the bf16
// rounding of the remainder (four products per value tile), about 2^-17,
// with c = rho_t . k_0.

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  i32x4 v = {(int)a, (int)b, (int)c, (int)d};
  return __builtin_bit_cast(f16x8, v);
}

// Two fp32 -> packed fp16 pair, rounded toward zero (a in the low half). Out
// of range values saturate to the largest finite fp16 instead of overflowing.
__device__ __forceinline__ f16x2 pack_f16_rtz(float a, float b) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// 8 bf16 -> 8 fp16. Exact for magnitudes in [2^-14, 65504] (fp16 keeps all 8
// significant bits of bf16 there); smaller ones lose bits below 2^-24.
__device__ __forceinline__ i32x4 bf16x8_to_f16x8(i32x4 x) {
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = (uint32_t)x[i];
    r[i] = __builtin_bit_cast(int, pack_f16_rtz(bf16_lo(w), bf16_hi(w)));
  }
  return r;
}

// Sum and max of x over the lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four
// lane groups that hold one query row), with the CDNA4 lane swaps
// (v_permlane16_swap / v_permlane32_swap: VALU, no LDS round trip). Each swap
// of x with itself leaves x_l and x_{l^16} (x_{l^32}) in the two results, in
// an order that depends on the lane, so every lane of a row gets the same
// (commutative) sum.
__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kWaves = 8;       // 16 rows per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 32;       // keys per block
constexpr int kNB = 2;          // key blocks per barrier
constexpr float kRescaleLog2 = 8.0f;
constexpr float kRefLog2 = 3.0f;       // block-max jump that moves the probe reference

// Key blocks staged per barrier: kNB consecutive blocks with one key range
// per workgroup (NS = 1), else one block of each of the NS key ranges.
constexpr int slots_for(int NS) { return NS == 1 ? kNB : NS; }

template <int D>
struct Pre {
  static constexpr int ROWB = D * 2;                  // bytes per bf16 row
  // Padded LDS row strides (bytes). V rows are read by the transposing load
  // 8 rows x 32 bytes at a time, which a 32-byte pad spreads over the banks.
  // K rows are read 16 rows x 16 bytes at a time. A 16-byte pad serves those
  // reads, yet left bank conflicts in about 28% of the LDS-active cycles; with
  // the 32-byte pad the counter reads zero and both prefills run about 1%
  // faster, so both tiles use it.
  static constexpr int LSTR = ROWB + 32;
  static constexpr int VSTR = ROWB + 32;
  static constexpr int KST = D / 32;                  // k-steps of the score MFMA
  static constexpr int DPL = D / 16;                  // N-tiles of the value MFMA
  static constexpr int PIECES = kKeys * ROWB / 16;    // 16-byte pieces per K (or V) tile
  static constexpr int PPT = 2 * PIECES / kThreads;   // pieces per thread per block (K and V)
  static constexpr int TILE = kKeys * VSTR;           // bytes of one staged K or V tile
};

// One row block (16 TL query rows starting at rb 16 TL) of one (b, h). With
// NS > 1 (short chunks) the first NS TL waves are NS key ranges times TL
// tiles of 16 rows: each streams one range of the keys its rows see, and the
// ranges' partial states merge in LDS at the end; any further waves only
// help stage the key blocks. TRAIN
// (the training forward, which also writes mu_v and the row statistics the
// backward recomputes the weights from) contracts the weights as split bf16
// pairs against bf16 V; otherwise they are rounded once to fp16 against fp16 V.
template <int D, bool TRAIN, int NS, int TL>
__device__ __forceinline__ void prefill_rows(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ past_lens, float* __restrict__ out, float* __restrict__ mu_out,
    float4* __restrict__ stats, int H_q, int H_kv, int G, int T, int S_max, float scale_log2, int rb,
    int h, int b, char (&kv_lds)[2 * slots_for(NS)][2][Pre<D>::TILE]) {
  using P = Pre<D>;
  static_assert(NS == 1 || !TRAIN, "key ranges are split in the inference form only");
  static_assert(NS * TL <= kWaves && (NS > 1 || TL == kWaves), "wave roles");
  constexpr int SLOTS = slots_for(NS);
  constexpr int TILES = TL;          // 16-row tiles
  constexpr int ROWS = 16 * TILES;   // query rows of the workgroup
  // the range merge reuses the stage buffers: per-row states of every range
  // and the accumulators of ranges 1.. (2 DPL f32x4 per lane)
  static_assert(NS == 1 || (NS * TILES * 16 * 4 + (NS - 1) * TILES * 64 * 2 * P::DPL * 4) * 4 <=
                               (int)sizeof(kv_lds), "range merge fits in the stage buffers");
  const int hk = h / G;
  // Row t of this chunk sits at position past + t of the sequence and sees
  // keys 0 .. past + t of the cache; rows t >= n are zero.
  const int past = past_lens ? min(max(past_lens[b], 0), S_max) : 0;
  const int n = min(min(max(seq_lens[b], 0), T), S_max - past);
  const int R0 = rb * ROWS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int rt = wave % TILES;  // this wave's row tile
  const int sp = wave / TILES;  // this wave's key range (NS and up: staging only)
  const int lane = tid & 63;
  const int g = lane >> 4;     // lane group
  const int c = lane & 15;     // query row within the wave (score layout) / output column
  const int wrow0 = R0 + 16 * rt;
  const int my_row = wrow0 + c;

  const size_t qbase = ((size_t)b * H_q + h) * (size_t)T * D;
  float* obase = out + qbase;

  if (R0 >= n) {  // whole block past the sequence: zeros
    for (int i = tid; i < ROWS * D / 4; i += kThreads) {
      const int r = R0 + i / (D / 4);
      if (r < T) {
        reinterpret_cast<float4*>(obase + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
        if (mu_out)
          reinterpret_cast<float4*>(mu_out + qbase + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (stats)
      for (int r = R0 + tid; r < min(R0 + ROWS, T); r += kThreads)
        stats[((size_t)b * H_q + h) * T + r] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }

  // q and rho operands (B of the transposed score MFMA): row my_row, dims
  // 32 kk + 8 g + (0..7). Rows past the sequence contribute zeros.
  bf16x8 qop[P::KST], rop[P::KST];
  {
    const bool live = my_row < n;
    const __bf16* qp = q + qbase + (size_t)(live ? my_row : 0) * D + 8 * g;
    const __bf16* rp = rho + qbase + (size_t)(live ? my_row : 0) * D + 8 * g;
    // With a negative scale, q is negated (exact in bf16) so that the scale
    // applied below is non-negative and the max of the raw scores gives the
    // max of the scaled ones.
    const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < P::KST; ++kk) {
      uint4 a = *reinterpret_cast<const uint4*>(qp + 32 * kk);
      uint4 r = *reinterpret_cast<const uint4*>(rp + 32 * kk);
      if (!live) a = r = uint4{0u, 0u, 0u, 0u};
      a.x ^= qsign;
      a.y ^= qsign;
      a.z ^= qsign;
      a.w ^= qsign;
      qop[kk] = as_bf16x8(a.x, a.y, a.z, a.w);
      rop[kk] = as_bf16x8(r.x, r.y, r.z, r.w);
    }
  }

  const float sl = fabsf(scale_log2);  // scale in log2 units, applied to the raw scores
  const size_t kvslice = ((size_t)b * H_kv + hk) * (size_t)S_max * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + kvslice, (uint32_t)(past + n) * P::ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + kvslice, (uint32_t)(past + n) * P::ROWB);

  // keys this workgroup needs, and this wave's number of key blocks
  const int wg_keys = past + min(R0 + ROWS, n);
  const int nkb = (wg_keys + kKeys - 1) / kKeys;
  const int wave_nkb = wrow0 < n ? (past + min(wrow0 + 15, n - 1)) / kKeys + 1 : 0;
  // key ranges: blocks [i spl, (i + 1) spl) form range i
  const int spl = (nkb + NS - 1) / NS;
  const int my_pos = past + my_row;  // last key this lane's row sees

  // Tile pieces of this thread (16 bytes each). With PPT >= 2 the first half
  // of a thread's pieces are K and the rest V; with PPT == 1 (d = 64) the
  // first half of the waves load K and the rest V. Either way the choice is
  // wave-uniform, so the buffer descriptor stays in scalar registers.
  auto piece = [&](int i, int& which, int& idx) {
    if constexpr (P::PPT >= 2) {
      which = i < P::PPT / 2 ? 0 : 1;
      idx = tid + kThreads * (i % (P::PPT / 2));
    } else {
      which = __builtin_amdgcn_readfirstlane(tid / (kThreads / 2));
      idx = tid % (kThreads / 2);
    }
  };
  // register stages: one (NS = 1), or two with split key ranges, whose
  // steps contract only one block per wave and so cover less load latency
  constexpr int NREG = NS == 1 ? 1 : 2;
  i32x4 stage[NREG][SLOTS][P::PPT];
  auto load_tile = [&](int kb, i32x4 (&dst)[P::PPT]) {
#pragma unroll
    for (int i = 0; i < P::PPT; ++i) {
      int which, idx;
      piece(i, which, idx);
      const int r = idx / (P::ROWB / 16);
      const int c16 = idx % (P::ROWB / 16);
      const uint32_t off = (uint32_t)(kb * kKeys + r) * P::ROWB + c16 * 16;
      dst[i] = __builtin_amdgcn_raw_buffer_load_b128(which ? vrs : krs, off, 0, 0);
    }
  };
  auto store_tile = [&](int buf, const i32x4 (&src)[P::PPT]) {
#pragma unroll
    for (int i = 0; i < P::PPT; ++i) {
      int which, idx;
      piece(i, which, idx);
      const int r = idx / (P::ROWB / 16);
      const int c16 = idx % (P::ROWB / 16);
      // without TRAIN, V is staged as fp16 (the value MFMAs take fp16 weights)
      const i32x4 val = (!TRAIN && which) ? bf16x8_to_f16x8(src[i]) : src[i];
      *reinterpret_cast<i32x4*>(&kv_lds[buf][which][r * (which ? P::VSTR : P::LSTR) + c16 * 16]) = val;
    }
  };

  f32x4 accA[P::DPL], accC[P::DPL];
#pragma unroll
  for (int j = 0; j < P::DPL; ++j) {
    accA[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accC[j] = accA[j];
  }
  float m = -INFINITY;  // running max (log2 units) of row my_row
  float lsum = 0.f;     // this lane's part of l (its 8 keys per block)
  float bsum = 0.f;     // this lane's part of Bs
  f32x4 rinit = {0.f, 0.f, 0.f, 0.f};  // start of the rho . k accumulators: -rho_t . k_0

  // Training forward, weights as split bf16 pairs: the reference c is
  // rho_t . k_0 (taken on block 0), the row max moves lazily (by more than
  // 2^8), and e and e (r - c) reach the value MFMAs as a bf16 high part plus
  // the bf16 rounding of the remainder (four products per value tile), so the
  // fp32 weights survive the contraction to about 2^-17: mu_v and the row
  // statistics feed the gradients, where the 2^-12 of one fp16 rounding
  // would use up most of the error bar.
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  auto contract_split = [&](int kb, f32x4 (&sc)[2], f32x4 (&rc)[2], const i16x4 (&vr)[P::DPL][2]) {
    if (kb == 0) {
      const float cref = __shfl(rc[0][0], c);  // key 0 sits in lane (0, c), slot 0
      rinit = f32x4{-cref, -cref, -cref, -cref};
#pragma unroll
      for (int T2 = 0; T2 < 2; ++T2) rc[T2] -= cref;
    }
    float mx = -INFINITY;
    const bool diag = kb * kKeys + kKeys - 1 > past + wrow0;
    if (diag) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb * kKeys + 16 * (e >> 2) + 4 * g + (e & 3);
        mx = fmaxf(mx, key <= my_pos ? sc[e >> 2][e & 3] : -INFINITY);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc[e >> 2][e & 3]);
    }
    mx *= sl;
    // Lazy rescale: each lane checks its own 8 keys; the row max (two
    // exchanges) is formed only when some lane exceeds the bound.
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleLog2)) {
      mx = row_max4(mx);
      const bool need = mx > m + kRescaleLog2;
      const float mnew = need ? mx : m;
      const float alpha = need ? exp2f(m - mnew) : 1.0f;
      m = mnew;
      lsum *= alpha;
      bsum *= alpha;
      float arow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) arow[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int j = 0; j < P::DPL; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accA[j][i] *= arow[i];
          accC[j][i] *= arow[i];
        }
    }
    float ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e >> 2][e & 3], sl, -m));
    if (diag) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb * kKeys + 16 * (e >> 2) + 4 * g + (e & 3);
        ev[e] = key <= my_pos ? ev[e] : 0.f;
      }
    }
    uint32_t phw[4], plw[4], qhw[4], qlw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float e0 = ev[2 * u];
      const float e1 = ev[2 * u + 1];
      const float f0 = e0 * rc[u >> 1][(2 * u) & 3];
      const float f1 = e1 * rc[u >> 1][(2 * u + 1) & 3];
      lsum += e0 + e1;
      bsum += f0 + f1;
      const uint32_t ph = pack_bf16(e0, e1);
      const uint32_t qh = pack_bf16(f0, f1);
      phw[u] = ph;
      qhw[u] = qh;
      plw[u] = pack_bf16(e0 - bf16_lo(ph), e1 - bf16_hi(ph));
      qlw[u] = pack_bf16(f0 - bf16_lo(qh), f1 - bf16_hi(qh));
    }
    const bf16x8 a_ph = as_bf16x8(phw[0], phw[1], phw[2], phw[3]);
    const bf16x8 a_pl = as_bf16x8(plw[0], plw[1], plw[2], plw[3]);
    const bf16x8 a_qh = as_bf16x8(qhw[0], qhw[1], qhw[2], qhw[3]);
    const bf16x8 a_ql = as_bf16x8(qlw[0], qlw[1], qlw[2], qlw[3]);
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vr[j][0], vr[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
      accA[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ph, vop, accA[j], 0, 0, 0);
      accA[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_pl, vop, accA[j], 0, 0, 0);
      accC[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_qh, vop, accC[j], 0, 0, 0);
      accC[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ql, vop, accC[j], 0, 0, 0);
    }
  };

  // Contracts key block kb (LDS buffer buf) into this wave's accumulators.
  auto contract = [&](int kb, int buf) {
    // ---- transposed scores: lane (g, c) holds row my_row, keys 16 T + 4 g + i.
    // The rho . k accumulators start at -c (c = rho_t . k_0, known from block
    // 0 on), so they come out already relative to the reference.
    // Issue order (pinned by scheduling barriers): every K operand read, then
    // the score MFMAs, then every V operand read, so the V reads are in flight
    // while the scores finish and the softmax runs, instead of each value
    // MFMA waiting on its own LDS round trip.
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    bf16x8 kop[2][P::KST];
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2) {
      const char* krow = &kv_lds[buf][0][(16 * T2 + c) * P::LSTR + 16 * g];
#pragma unroll
      for (int kk = 0; kk < P::KST; ++kk)
        kop[T2][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(krow + 64 * kk));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[2], rc[2];
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2) {
      sc[T2] = f32x4{0.f, 0.f, 0.f, 0.f};
      rc[T2] = rinit;
#pragma unroll
      for (int kk = 0; kk < P::KST; ++kk) {
        sc[T2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[T2][kk], qop[kk], sc[T2], 0, 0, 0);
        rc[T2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[T2][kk], rop[kk], rc[T2], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // V operands. The B operand of N-tile j (dims 16 j .. 16 j + 15) in lane
    // (g, c) is V at dim 16 j + c for key slots e = 0..7 (keys 16 (e / 4) +
    // 4 g + e % 4). Each half (e < 4, e >= 4) comes from one transposing LDS
    // load: within a group of 16 lanes, lane 4 a + b receives element b of
    // the 8-byte pieces addressed by lanes a, a + 4, a + 8 and a + 12, so lane
    // s of group g addresses key 16 h + 4 g + s / 4 at dims 16 j + 4 (s % 4)
    // .. + 3.
    const char* vbase = &kv_lds[buf][1][(4 * g + (c >> 2)) * P::VSTR + 8 * (c & 3)];
    i16x4 vr[P::DPL][2];
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      vr[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 32 * j));
      vr[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + 32 * j + 16 * P::VSTR));
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (TRAIN) {
      contract_split(kb, sc, rc, vr);
      return;
    }

    // Raw scores; masked keys are -inf on the block that reaches past this
    // wave's first row. The weights are exp2(sl s - m), with the scaled max
    // sl max(s) (sl >= 0).
    float mx = -INFINITY;
    const bool diag = kb * kKeys + kKeys - 1 > past + wrow0;
    if (diag) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb * kKeys + 16 * (e >> 2) + 4 * g + (e & 3);
        mx = fmaxf(mx, key <= my_pos ? sc[e >> 2][e & 3] : -INFINITY);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc[e >> 2][e & 3]);
    }
    mx *= sl;

    // Reference moves (rare, wave-uniform branch): taken on the first block
    // and whenever some lane's block max exceeds its row's reference max m by
    // more than 2^3 (a key that now outweighs the reference key 8-fold).
    //  - Lazy rescale: m only has to bound every weight exp2(x - m) by 2^8
    //    (fp16 holds the weights), so it moves to the row max only past that.
    //  - Probe reference: c moves to the running weighted mean of r (this
    //    block included), so the products e (r - c), rounded once to fp16,
    //    stay small next to the weights that dominate the row. The shift is
    //    exact: Bs -> Bs - delta l and C -> C - delta A.
    const bool moved = __builtin_amdgcn_ballot_w64(mx > m + kRefLog2) != 0;
    float alpha = 1.0f;
    if (moved) {  // VALU only: the row max through lane swaps
      mx = row_max4(mx);
      const bool need = mx > m + kRescaleLog2;
      const float mnew = need ? mx : m;
      alpha = need ? exp2f(m - mnew) : 1.0f;
      m = mnew;
      lsum *= alpha;
      bsum *= alpha;
    }
    float ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e >> 2][e & 3], sl, -m));
    if (diag) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb * kKeys + 16 * (e >> 2) + 4 * g + (e & 3);
        ev[e] = key <= my_pos ? ev[e] : 0.f;
      }
    }
    if (moved) {
      // One pass over the accumulators for both moves, with one broadcast
      // round trip: A <- alpha A and C <- alpha (C - delta A).
      float le = 0.f, be = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        le += ev[e];
        be += ev[e] * rc[e >> 2][e & 3];
      }
      const float ltot = row_sum4(lsum + le);
      const float btot = row_sum4(bsum + be);
      // Any reference is exact. A row with no visible key yet (in a key range
      // after the first, the rows before its first key) keeps its reference.
      const float delta = ltot > 0.f ? btot * __builtin_amdgcn_rcpf(ltot) : 0.f;
      bsum -= delta * lsum;
      rinit -= delta;
#pragma unroll
      for (int T2 = 0; T2 < 2; ++T2) rc[T2] -= delta;
      // accumulator rows 4 g + i belong to the lanes whose column is 4 g + i
      float arow[4], drow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        arow[i] = __shfl(alpha, 4 * g + i);
        drow[i] = __shfl(delta, 4 * g + i);
      }
#pragma unroll
      for (int j = 0; j < P::DPL; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accC[j][i] = __builtin_fmaf(-drow[i], accA[j][i], accC[j][i]) * arow[i];
          accA[j][i] *= arow[i];
        }
    }

    // ---- weights e and e (r - c), each rounded once to fp16 (toward zero):
    // the A operands of the value MFMAs. l and Bs sum the rounded values, so
    // the weights that reach A and C are exactly those of l and Bs, and the
    // rounding only perturbs each weight by less than 2^-10 of itself instead of
    // leaving A out of step with l.
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    uint32_t pw[4], fw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float e0 = ev[2 * u];
      const float e1 = ev[2 * u + 1];
      const f16x2 ph = pack_f16_rtz(e0, e1);
      const f16x2 fh = pack_f16_rtz(e0 * rc[u >> 1][(2 * u) & 3], e1 * rc[u >> 1][(2 * u + 1) & 3]);
      lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
      bsum = __builtin_amdgcn_fdot2(fh, ones, bsum, false);
      pw[u] = __builtin_bit_cast(uint32_t, ph);
      fw[u] = __builtin_bit_cast(uint32_t, fh);
    }
    const f16x8 a_p = as_f16x8(pw[0], pw[1], pw[2], pw[3]);
    const f16x8 a_f = as_f16x8(fw[0], fw[1], fw[2], fw[3]);

    // ---- value MFMAs (V was staged as fp16)
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      const f16x8 vop = __builtin_bit_cast(f16x8, __builtin_shufflevector(vr[j][0], vr[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
      accA[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_p, vop, accA[j], 0, 0, 0);
      accC[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_f, vop, accC[j], 0, 0, 0);
    }
  };

  // Pipeline, one barrier per step of SLOTS staged blocks: the blocks of
  // step s are contracted from LDS buffers pb .. pb + SLOTS - 1 while the
  // next step's blocks go from registers into the other buffers and the step
  // after them is loaded from HBM into the registers just freed (each load
  // has a step of contraction to land). With one key range (NS = 1) a step
  // holds kNB consecutive blocks: two blocks per barrier halve the barriers
  // and the LDS operand waits that follow each one (causal prefill about 2%
  // faster than one block per barrier; three or four blocks gave no more).
  // With NS ranges a step holds the s-th block of each range, and each wave
  // contracts its own range's. Loads and stores run unconditionally: loads
  // past the sequence are range-checked to zeros without touching memory.
  // The loop is unrolled by two steps so that every buffer index is static.
  auto block_of = [&](int st, int i) { return NS == 1 ? st * SLOTS + i : i * spl + st; };
  const int nsteps = NS == 1 ? (nkb + SLOTS - 1) / SLOTS : spl;
  // Step st: contract the blocks of step st from LDS buffers pb ..; move the
  // register stage holding step st + 1 into the other buffers; refill that
  // stage with step st + 1 + NREG.
  auto step = [&](int st, int pb, i32x4 (&rs)[SLOTS][P::PPT]) {
    if constexpr (NS == 1) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        if (block_of(st, i) < wave_nkb) contract(block_of(st, i), pb + i);
    } else {  // one contraction, from this wave's range's buffer (wave-uniform)
      const int kb = block_of(st, sp);
      if (sp < NS && kb < wave_nkb && st < spl) contract(kb, pb + sp);
    }
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) store_tile((pb ^ SLOTS) + i, rs[i]);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) load_tile(block_of(st + 1 + NREG, i), rs[i]);
    __syncthreads();
  };
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) load_tile(block_of(0, i), stage[0][i]);
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) store_tile(i, stage[0][i]);
#pragma unroll
  for (int r = 0; r < NREG; ++r)
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) load_tile(block_of(1 + r, i), stage[(1 + r) % NREG][i]);
  __syncthreads();
  // Both steps of an iteration are unconditional and an odd last step runs
  // after the loop: the loop is then entered only with the stages in one age
  // order, so the load waits count just the loads a store needs.
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, 0, stage[1 % NREG]);
    step(st + 1, SLOTS, stage[0]);
  }
  if (st < nsteps) step(st, 0, stage[1 % NREG]);

  // ---- finalise: row totals of l and Bs, moved to the output layout
  float ltot = row_sum4(lsum);
  float btot = row_sum4(bsum);
  if constexpr (NS > 1) {
    // Merge the key ranges of each row tile into the wave of range 0. Each
    // range's state: per row (score layout) m, l, Bs and the reference c;
    // per lane the accumulators (output layout). A range without keys has
    // l = 0 and weight 0; the reference becomes range 0's (key 0 is in it).
    float* f = reinterpret_cast<float*>(&kv_lds[0][0][0]);
    float* rstat = f;                               // [NS][TILES][16 rows][4]
    float* rvec = f + NS * TILES * 16 * 4;          // [NS - 1][TILES][64 lanes][2 DPL 4]
    constexpr int VW = 2 * P::DPL * 4;
    if (g == 0 && sp < NS) {
      float* st4 = rstat + ((sp * TILES + rt) * 16 + c) * 4;
      st4[0] = m;
      st4[1] = ltot;
      st4[2] = btot;
      st4[3] = -rinit[0];
    }
    if (sp > 0 && sp < NS) {
      float* v = rvec + (((sp - 1) * TILES + rt) * 64 + lane) * VW;
#pragma unroll
      for (int j = 0; j < P::DPL; ++j) {
        *reinterpret_cast<f32x4*>(v + 8 * j) = accA[j];
        *reinterpret_cast<f32x4*>(v + 8 * j + 4) = accC[j];
      }
    }
    __syncthreads();
    if (sp > 0) return;
    // per-row weights of every range, in both layouts: row c (scalars) and
    // rows 4 g + i (accumulators)
    auto row_weights = [&](int r, float& M, float& c0) {
      M = -INFINITY;
      c0 = rstat[((0 * TILES + rt) * 16 + r) * 4 + 3];
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const float* st4 = rstat + ((s2 * TILES + rt) * 16 + r) * 4;
        M = st4[1] > 0.f ? fmaxf(M, st4[0]) : M;
      }
    };
    {
      float M, c0;
      row_weights(c, M, c0);
      float l = 0.f, bs = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const float* st4 = rstat + ((s2 * TILES + rt) * 16 + c) * 4;
        const float al = st4[1] > 0.f ? exp2f(st4[0] - M) : 0.f;
        l += al * st4[1];
        bs += al * (st4[2] + (st4[3] - c0) * st4[1]);
      }
      ltot = l;
      btot = bs;
      m = M;  // the training statistics are not kept with several ranges
    }
    // accumulators (rows 4 g + i): this wave's own range first, then one
    // range at a time (a rolled loop, so that only one range's values are
    // held in registers at once)
    float M4[4], c04[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      row_weights(4 * g + i, M4[i], c04[i]);
      const float* st4 = rstat + ((0 * TILES + rt) * 16 + 4 * g + i) * 4;
      const float al = st4[1] > 0.f ? exp2f(st4[0] - M4[i]) : 0.f;
      const float sh = st4[3] - c04[i];
#pragma unroll
      for (int j = 0; j < P::DPL; ++j) {
        accC[j][i] = al * (accC[j][i] + sh * accA[j][i]);
        accA[j][i] = al * accA[j][i];
      }
    }
#pragma unroll 1
    for (int s2 = 1; s2 < NS; ++s2) {
      float al[4], sh[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* st4 = rstat + ((s2 * TILES + rt) * 16 + 4 * g + i) * 4;
        al[i] = st4[1] > 0.f ? exp2f(st4[0] - M4[i]) : 0.f;
        sh[i] = st4[3] - c04[i];
      }
      const float* v = rvec + (((s2 - 1) * TILES + rt) * 64 + lane) * VW;
#pragma unroll
      for (int j = 0; j < P::DPL; ++j) {
        const f32x4 aw = *reinterpret_cast<const f32x4*>(v + 8 * j);
        const f32x4 cw = *reinterpret_cast<const f32x4*>(v + 8 * j + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accA[j][i] += al[i] * aw[i];
          accC[j][i] += al[i] * (cw[i] + sh[i] * aw[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = 4 * g + i;  // row within the wave held by this lane's accumulators
    const float l = __shfl(ltot, lr);
    const float bsr = __shfl(btot, lr);
    // training mode: the row's m and reference c live in the lanes whose column is lr
    const float mrow = __shfl(m, lr);
    const float crow = -__shfl(rinit[0], lr);
    const int t = wrow0 + lr;
    if (t >= T) continue;
    float ov[P::DPL];
    const bool live = t < n;
    const float inv_l = live ? 1.f / l : 0.f;
    const float gain = 1.f + bsr * inv_l;
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) ov[j] = live ? (accA[j][i] * gain - accC[j][i]) * inv_l : 0.f;
    float* dst = obase + (size_t)t * D + c;  // column c of N-tile j is dim 16 j + c
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) dst[16 * j] = ov[j];
    if (mu_out) {  // mu_v = A / l
      float* mdst = mu_out + qbase + (size_t)t * D + c;
#pragma unroll
      for (int j = 0; j < P::DPL; ++j) mdst[16 * j] = accA[j][i] * inv_l;
    }
    // (log2-sum-exp of the scaled scores, reference c = rho . k_0, Bs / l = rbar - c)
    if (stats && c == 0)
      stats[((size_t)b * H_q + h) * T + t] =
          live ? float4{mrow + __builtin_log2f(l), crow, bsr * inv_l, 0.f} : float4{0.f, 0.f, 0.f, 0.f};
  }
}

// With one key range (NS = 1), workgroup x handles row blocks nrb - 1 - x
// and x of one (b, h): under the causal mask their key counts add up to the
// same total for every x, so all workgroups carry equal work and the short
// early row blocks never form a tail of their own. Short chunks (NS > 1),
// whose row blocks all see about the same keys, take one row block per
// workgroup, so that a few rows per head still fill the chip.
template <int D, bool TRAIN, int NS, int TL>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ past_lens, float* __restrict__ out, float* __restrict__ mu_out,
    float4* __restrict__ stats, int H_q, int H_kv, int G, int T, int S_max, float scale_log2) {
  // [buffer][K, V]
  __shared__ __attribute__((aligned(16))) char kv_lds[2 * slots_for(NS)][2][Pre<D>::TILE];
  const int nrb = (T + 16 * TL - 1) / (16 * TL);
  // Workgroups are dealt to the 8 XCDs in linear order. Remap so that each
  // XCD takes a contiguous range of (sequence, head, row-block pair) tiles:
  // the query heads of one KV head are adjacent, so the workgroups running at
  // the same time on an XCD mostly share one K/V slice in that XCD's L2.
  int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const unsigned long long total = (unsigned long long)gridDim.x * gridDim.y * gridDim.z;
  if (total < (1ull << 31) && total % 8u == 0u) {
    const unsigned npairs = gridDim.x, tot = (unsigned)total;
    const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned L = (lin % 8u) * (tot / 8u) + lin / 8u;
    x = (int)(L % npairs);
    h = (int)((L / npairs) % gridDim.y);
    b = (int)(L / (npairs * gridDim.y));
  }
  if constexpr (NS > 1) {
    prefill_rows<D, TRAIN, NS, TL>(q, rho, kc, vc, seq_lens, past_lens, out, mu_out, stats, H_q,
                                   H_kv, G, T, S_max, scale_log2, x, h, b, kv_lds);
  } else {
    prefill_rows<D, TRAIN, NS, TL>(q, rho, kc, vc, seq_lens, past_lens, out, mu_out, stats, H_q,
                                   H_kv, G, T, S_max, scale_log2, nrb - 1 - x, h, b, kv_lds);
    if (x != nrb - 1 - x) {
      __syncthreads();
      prefill_rows<D, TRAIN, NS, TL>(q, rho, kc, vc, seq_lens, past_lens, out, mu_out, stats, H_q,
                                     H_kv, G, T, S_max, scale_log2, x, h, b, kv_lds);
    }
  }
}

template <int D, bool TRAIN, int NS, int TL>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int nrb = (a.T + 16 * TL - 1) / (16 * TL);
  // one row block per workgroup with split key ranges, else pairs (heavy + light)
  dim3 grid(NS > 1 ? nrb : (nrb + 1) / 2, a.H_q, a.B);
  hipLaunchKernelGGL((prefill_kernel<D, TRAIN, NS, TL>), grid, dim3(kThreads), 0, st,
                     static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.rho),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v), a.seq_lens,
                     a.past_lens, a.out, a.mu_out, static_cast<float4*>(a.stats), a.H_q, a.H_kv,
                     a.G, a.T, a.S_max, a.scale * kLog2e);
  return hipGetLastError();
}

// Inference forms by chunk length: up to 32 rows, four key ranges of one
// 16-row tile (half the waves contract, all of them stage keys); up to 64,
// four ranges of two tiles; up to 256, two ranges of four tiles (64-row
// blocks: at 8 sequences of 16 heads, 256 to 512 workgroups where paired
// 128-row blocks give 128); longer chunks, one range of eight tiles.
template <int D>
hipError_t launch_prefill_infer(const PrefillArgs& a, hipStream_t st) {
  if (a.T <= 32) return launch_prefill_t<D, false, 4, 1>(a, st);
  if (a.T <= 64) return launch_prefill_t<D, false, 4, 2>(a, st);
  if (a.T <= 256) return launch_prefill_t<D, false, 2, 4>(a, st);
  return launch_prefill_t<D, false, 1, kWaves>(a, st);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.mu_out != nullptr)  // training forward
    return a.d == 64 ? launch_prefill_t<64, true, 1, kWaves>(a, st)
                     : launch_prefill_t<128, true, 1, kWaves>(a, st);
  return a.d == 64 ? launch_prefill_infer<64>(a, st) : launch_prefill_infer<128>(a, st);
}

}  // namespace parallax
