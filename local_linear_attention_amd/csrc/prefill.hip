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
// The per-row reference c_t = rho_t.k_0 cancels exactly (it shifts Bs by
// c l and C by c A) and keeps a large common offset of rho.k out of the
// accumulated products.
//
// Tiling. A workgroup of 8 waves owns 128 query rows of one (b, h); each wave
// owns 16 rows, so a wave needs about 204 registers and two waves share each
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
// [e; e r] V with e and e r each split into a bf16 high part and the bf16
// rounding of the remainder (four products), so the fp32 weights reach the
// bf16 contraction to about 2^-17. The V operand (key slots down, dims
// across) comes straight from the row-major V tile through the CDNA4
// transposing LDS load (ds_read_b64_tr_b16), so no lane shuffles V in
// registers; output column c of N-tile j is dim 16 j + c. Softmax rescaling
// is lazy (only when a block's max exceeds the running reference by more than
// 2^8). Each workgroup handles a heavy (late) and a light (early) row block,
// so every workgroup carries the same causal work.

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kRows = 128;      // query rows per workgroup
constexpr int kWaves = 8;       // 16 rows per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 32;       // keys per block
constexpr int kNB = 2;          // key blocks per barrier
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Pre {
  static constexpr int ROWB = D * 2;                  // bytes per bf16 row
  // Padded LDS row strides (bytes): K rows are read 16 rows x 16 bytes at a
  // time (a 16-byte pad spreads them over all banks); V rows are read by the
  // transposing load 8 rows x 32 bytes at a time (a 32-byte pad does).
  static constexpr int LSTR = ROWB + 16;
  static constexpr int VSTR = ROWB + 32;
  static constexpr int KST = D / 32;                  // k-steps of the score MFMA
  static constexpr int DPL = D / 16;                  // N-tiles of the value MFMA
  static constexpr int PIECES = kKeys * ROWB / 16;    // 16-byte pieces per K (or V) tile
  static constexpr int PPT = 2 * PIECES / kThreads;   // pieces per thread per block (K and V)
  static constexpr int TILE = kKeys * VSTR;           // bytes of one staged K or V tile
};

// One row block (128 query rows starting at rb * 128) of one (b, h).
template <int D>
__device__ __forceinline__ void prefill_rows(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ past_lens, float* __restrict__ out, float* __restrict__ mu_out,
    float4* __restrict__ stats, int H_q, int H_kv, int G, int T, int S_max, float scale_log2, int rb,
    int h, int b, char (&kv_lds)[2 * kNB][2][Pre<D>::TILE]) {
  using P = Pre<D>;
  const int hk = h / G;
  // Row t of this chunk sits at position past + t of the sequence and sees
  // keys 0 .. past + t of the cache; rows t >= n are zero.
  const int past = past_lens ? min(max(past_lens[b], 0), S_max) : 0;
  const int n = min(min(max(seq_lens[b], 0), T), S_max - past);
  const int R0 = rb * kRows;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int g = lane >> 4;     // lane group
  const int c = lane & 15;     // query row within the wave (score layout) / output column
  const int wrow0 = R0 + 16 * wave;
  const int my_row = wrow0 + c;

  const size_t qbase = ((size_t)b * H_q + h) * (size_t)T * D;
  float* obase = out + qbase;

  if (R0 >= n) {  // whole block past the sequence: zeros
    for (int i = tid; i < kRows * D / 4; i += kThreads) {
      const int r = R0 + i / (D / 4);
      if (r < T) {
        reinterpret_cast<float4*>(obase + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
        if (mu_out)
          reinterpret_cast<float4*>(mu_out + qbase + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (stats)
      for (int r = R0 + tid; r < min(R0 + kRows, T); r += kThreads)
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
  const int wg_keys = past + min(R0 + kRows, n);
  const int nkb = (wg_keys + kKeys - 1) / kKeys;
  const int wave_nkb = wrow0 < n ? (past + min(wrow0 + 15, n - 1)) / kKeys + 1 : 0;
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
  i32x4 stage[kNB][P::PPT];
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
      *reinterpret_cast<i32x4*>(&kv_lds[buf][which][r * (which ? P::VSTR : P::LSTR) + c16 * 16]) = src[i];
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

  // Contracts key block kb (LDS buffer buf) into this wave's accumulators.
  auto contract = [&](int kb, int buf) {
    // ---- transposed scores: lane (g, c) holds row my_row, keys 16 T + 4 g + i.
    // The rho . k accumulators start at -c (c = rho_t . k_0, known from block
    // 0 on), so they come out already relative to the reference.
    // Issue order (pinned by scheduling barriers): every K operand read, then
    // the score MFMAs, then every V operand read, so the V reads are in flight
    // while the scores finish and the softmax runs, instead of each value
    // MFMA waiting on its own LDS round trip.
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
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
    if (kb == 0) {
      const float cref = __shfl(rc[0][0], c);  // key 0 sits in lane (0, c), slot 0
      rinit = f32x4{-cref, -cref, -cref, -cref};
#pragma unroll
      for (int T2 = 0; T2 < 2; ++T2) rc[T2] -= cref;
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

    // Lazy rescale. The reference m of a row only has to bound every weight
    // exp2(x - m) by 2^8, so each lane checks its own 8 keys; the row max
    // (two exchanges) is formed only when some lane exceeds the bound.
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleLog2)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m + kRescaleLog2;
      const float mnew = need ? mx : m;
      const float alpha = need ? exp2f(m - mnew) : 1.0f;
      m = mnew;
      lsum *= alpha;
      bsum *= alpha;
      // accumulator rows 4 g + i belong to the lanes whose column is 4 g + i
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

    // ---- weights e and e (r - c) as packed bf16 high parts and the bf16
    // rounding of the remainders: the A operands of the value MFMAs
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

    // ---- value MFMAs
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vr[j][0], vr[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
      accA[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ph, vop, accA[j], 0, 0, 0);
      accA[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_pl, vop, accA[j], 0, 0, 0);
      accC[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_qh, vop, accC[j], 0, 0, 0);
      accC[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ql, vop, accC[j], 0, 0, 0);
    }
  };

  // Pipeline, one barrier per kNB blocks of keys: blocks kb .. kb + kNB - 1
  // are contracted from LDS buffers pb .. pb + kNB - 1 while the next kNB
  // blocks go from registers into the other buffers and the kNB blocks after
  // them are loaded from HBM into the registers just freed (each load has kNB
  // blocks of contraction to land). Two blocks per barrier halve the barriers
  // and the LDS operand waits that follow each one (causal prefill about 2%
  // faster than one block per barrier; three or four blocks gave no more).
  // Loads and stores run unconditionally: loads past the sequence are
  // range-checked to zeros without touching memory. The loop is unrolled by
  // two groups so that every buffer index is static.
  auto groupstep = [&](int kb, int pb) {
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      if (kb + i < wave_nkb) contract(kb + i, pb + i);
#pragma unroll
    for (int i = 0; i < kNB; ++i) store_tile((pb ^ kNB) + i, stage[i]);
#pragma unroll
    for (int i = 0; i < kNB; ++i) load_tile(kb + 2 * kNB + i, stage[i]);
    __syncthreads();
  };
#pragma unroll
  for (int i = 0; i < kNB; ++i) load_tile(i, stage[i]);
#pragma unroll
  for (int i = 0; i < kNB; ++i) store_tile(i, stage[i]);
#pragma unroll
  for (int i = 0; i < kNB; ++i) load_tile(kNB + i, stage[i]);
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2 * kNB) {
    groupstep(kb, 0);
    if (kb + kNB < nkb) groupstep(kb + kNB, kNB);
  }

  // ---- finalise: row totals of l and Bs, moved to the output layout
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  float btot = bsum + __shfl_xor(bsum, 16);
  btot += __shfl_xor(btot, 32);
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

// Workgroup x handles row blocks nrb - 1 - x and x of one (b, h): under the
// causal mask their key counts add up to the same total for every x, so all
// workgroups carry equal work and the short early row blocks never form a
// tail of their own.
template <int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ past_lens, float* __restrict__ out, float* __restrict__ mu_out,
    float4* __restrict__ stats, int H_q, int H_kv, int G, int T, int S_max, float scale_log2) {
  __shared__ __attribute__((aligned(16))) char kv_lds[2 * kNB][2][Pre<D>::TILE];  // [buffer][K, V]
  const int nrb = (T + kRows - 1) / kRows;
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
  prefill_rows<D>(q, rho, kc, vc, seq_lens, past_lens, out, mu_out, stats, H_q, H_kv, G, T, S_max,
                  scale_log2, nrb - 1 - x, h, b, kv_lds);
  if (x != nrb - 1 - x) {
    __syncthreads();
    prefill_rows<D>(q, rho, kc, vc, seq_lens, past_lens, out, mu_out, stats, H_q, H_kv, G, T, S_max,
                    scale_log2, x, h, b, kv_lds);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int nrb = (a.T + kRows - 1) / kRows;
  dim3 grid((nrb + 1) / 2, a.H_q, a.B);  // row blocks paired heavy + light
  if (a.d == 64) {
    hipLaunchKernelGGL((prefill_kernel<64>), grid, dim3(kThreads), 0, st,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.rho),
                       static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                       a.seq_lens, a.past_lens, a.out, a.mu_out, static_cast<float4*>(a.stats), a.H_q,
                       a.H_kv, a.G, a.T, a.S_max, a.scale * kLog2e);
  } else {
    hipLaunchKernelGGL((prefill_kernel<128>), grid, dim3(kThreads), 0, st,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.rho),
                       static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                       a.seq_lens, a.past_lens, a.out, a.mu_out, static_cast<float4*>(a.stats), a.H_q,
                       a.H_kv, a.G, a.T, a.S_max, a.scale * kLog2e);
  }
  return hipGetLastError();
}

}  // namespace parallax
