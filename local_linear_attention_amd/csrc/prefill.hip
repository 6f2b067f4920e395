// Parallax causal prefill on CDNA4 (gfx950).
//
// Row t of sequence b, query head h, sees keys 0..t of KV head h / G
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
// Tiling. A workgroup of 4 waves owns 128 query rows of one (b, h); each wave
// owns 32 rows. Key blocks of 32 keys are staged in double-buffered LDS (rows
// padded by 16 bytes against bank conflicts) and shared by the 4 waves; a
// block's global loads are issued two blocks before it is needed. Per wave
// and key block, v_mfma_f32_32x32x16_bf16 computes the transposed scores
// S^T = K Q^T and R^T = K rho^T, so lane l holds query row l % 32 for keys
// 8p + 4 (l / 32) + i (p, i = 0..3): the row max and sums are lane-local plus
// one exchange with lane l ^ 32, and those 8 + 8 keys are exactly the key
// slots lane l supplies as the A operand of the two 16-key value MFMAs. The
// value MFMA computes [e; e r] V with e and e r each split into a bf16 high
// part and the bf16 rounding of the remainder (four products), so the fp32
// weights reach the bf16 contraction to about 2^-17. Each lane reads V rows
// of its 8 key slots, d/32 contiguous dims each, from LDS and hands dim j of
// every row to N-tile j (output column c of tile j is dim (d/32) c + j), so V
// needs no transpose. Softmax rescaling is lazy (only when a block's max
// exceeds the running reference by more than 2^8). Heavy (late) row blocks
// are dispatched first.

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kRows = 128;        // query rows per workgroup
constexpr int kKeys = 32;         // keys per block
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Pre {
  static constexpr int ROWB = D * 2;             // bytes per bf16 row
  static constexpr int LSTR = ROWB + 16;         // padded LDS row stride (bytes)
  static constexpr int KST = D / 16;             // k-steps of the score MFMA
  static constexpr int NT = D / 32;              // value N-tiles = dims per lane column
  static constexpr int PIECES = kKeys * ROWB / 16;  // 16-byte pieces per K (or V) tile
  static constexpr int PPT = 2 * PIECES / 256;   // pieces per thread per block (K and V)
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ rho, const __bf16* __restrict__ kc,
    const __bf16* __restrict__ vc, const int32_t* __restrict__ seq_lens, float* __restrict__ out,
    int H_q, int H_kv, int G, int T, int S_max, float scale_log2) {
  using P = Pre<D>;
  __shared__ __attribute__((aligned(16))) char kv_lds[2][2][kKeys * P::LSTR];  // [buffer][K, V]
  __shared__ float row_lds[4][2][32];  // per wave: two per-row scalars
  static_assert(2 * 2 * kKeys * Pre<D>::LSTR + sizeof(float) * 256 <= 65536, "LDS budget");

  const int nrb = (T + kRows - 1) / kRows;
  const int rb = nrb - 1 - (int)blockIdx.x;  // late (heavy) row blocks first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / G;
  const int n = min(max(seq_lens[b], 0), T);  // rows t >= n are zero; keys j <= t < n
  const int R0 = rb * kRows;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;   // query row (score layout) / output column
  const int half = lane >> 5;
  const int wrow0 = R0 + 32 * wave;  // first row of this wave
  const int my_row = wrow0 + col;    // row of this lane in the score layout

  const size_t qbase = ((size_t)b * H_q + h) * (size_t)T * D;
  float* obase = out + qbase;

  if (R0 >= n) {  // whole block past the sequence: zeros
    for (int i = tid; i < kRows * D / 4; i += 256) {
      const int r = R0 + i / (D / 4);
      if (r < T) reinterpret_cast<float4*>(obase + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }

  // q and rho operands (B of the transposed score MFMA): row my_row, dims
  // 16 kk + 8 half + (0..7). Rows past the sequence contribute zeros.
  bf16x8 qop[P::KST], rop[P::KST];
  {
    const bool live = my_row < n;
    const __bf16* qp = q + qbase + (size_t)(live ? my_row : 0) * D + 8 * half;
    const __bf16* rp = rho + qbase + (size_t)(live ? my_row : 0) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < P::KST; ++kk) {
      uint4 a = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      uint4 c = *reinterpret_cast<const uint4*>(rp + 16 * kk);
      if (!live) a = c = uint4{0u, 0u, 0u, 0u};
      qop[kk] = as_bf16x8(a.x, a.y, a.z, a.w);
      rop[kk] = as_bf16x8(c.x, c.y, c.z, c.w);
    }
  }

  const size_t kvslice = ((size_t)b * H_kv + hk) * (size_t)S_max * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + kvslice, (uint32_t)n * P::ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + kvslice, (uint32_t)n * P::ROWB);

  // keys this workgroup needs, and this wave's last key block
  const int wg_keys = min(R0 + kRows, n);
  const int nkb = (wg_keys + kKeys - 1) / kKeys;
  const int wave_last_key = min(wrow0 + 31, n - 1);
  const int wave_nkb = wave_last_key >= 0 && wrow0 < n ? wave_last_key / kKeys + 1 : 0;

  // tile pieces of this thread (16 bytes each); two register stages so that a
  // block's loads are issued two blocks ahead
  i32x4 stage[2][P::PPT];
  // Pieces 0 .. PPT/2-1 of a thread are K, the rest V (a compile-time split,
  // so the buffer descriptor stays wave-uniform).
  auto load_tile = [&](int kb, i32x4 (&dst)[P::PPT]) {
#pragma unroll
    for (int i = 0; i < P::PPT; ++i) {
      const int idx = tid + 256 * (i % (P::PPT / 2));
      const int r = idx / (P::ROWB / 16);
      const int c16 = idx % (P::ROWB / 16);
      const uint32_t off = (uint32_t)(kb * kKeys + r) * P::ROWB + c16 * 16;
      dst[i] = __builtin_amdgcn_raw_buffer_load_b128(i < P::PPT / 2 ? krs : vrs, off, 0, 0);
    }
  };
  auto store_tile = [&](int buf, const i32x4 (&src)[P::PPT]) {
#pragma unroll
    for (int i = 0; i < P::PPT; ++i) {
      const int idx = tid + 256 * (i % (P::PPT / 2));
      const int r = idx / (P::ROWB / 16);
      const int c16 = idx % (P::ROWB / 16);
      *reinterpret_cast<i32x4*>(&kv_lds[buf][i < P::PPT / 2 ? 0 : 1][r * P::LSTR + c16 * 16]) = src[i];
    }
  };

  f32x16_t accA[P::NT], accC[P::NT];
#pragma unroll
  for (int j = 0; j < P::NT; ++j) {
    accA[j] = f32x16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    accC[j] = accA[j];
  }
  float m = -INFINITY;  // running max (log2 units) of row my_row
  float lsum = 0.f;     // this lane's part of l (its 16 keys per block)
  float bsum = 0.f;     // this lane's part of Bs
  float cref = 0.f;     // rho_t . k_0

  // Contracts key block kb (LDS buffer buf) into this wave's accumulators.
  auto contract = [&](int kb, int buf) {
    // ---- transposed scores: lane holds row my_row, keys 8 (r / 4) + 4 half + r % 4
    f32x16_t sacc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    f32x16_t racc = sacc;
    const char* krow = &kv_lds[buf][0][col * P::LSTR + 16 * half];
#pragma unroll
    for (int kk = 0; kk < P::KST; ++kk) {
      const i32x4 kw = *reinterpret_cast<const i32x4*>(krow + 32 * kk);
      const bf16x8 kop = __builtin_bit_cast(bf16x8, kw);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], sacc, 0, 0, 0);
      racc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, rop[kk], racc, 0, 0, 0);
    }
    if (kb == 0) cref = __shfl(racc[0], col);  // key 0 sits in lane col, slot 0

    float x[16];
    float mx = -INFINITY;
    if (kb * kKeys + kKeys - 1 > wrow0) {  // diagonal block: causal mask
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * kKeys + 8 * (r >> 2) + 4 * half + (r & 3);
        x[r] = key <= my_row ? sacc[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = sacc[r] * scale_log2;
        mx = fmaxf(mx, x[r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    const bool need = mx > m + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mnew = need ? mx : m;
      const float alpha = need ? exp2f(m - mnew) : 1.0f;
      m = mnew;
      lsum *= alpha;
      bsum *= alpha;
      if (half == 0) row_lds[wave][0][col] = alpha;
      __builtin_amdgcn_wave_barrier();
      float arow[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) arow[r] = row_lds[wave][0][8 * (r >> 2) + 4 * half + (r & 3)];
#pragma unroll
      for (int j = 0; j < P::NT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          accA[j][r] *= arow[r];
          accC[j][r] *= arow[r];
        }
      __builtin_amdgcn_wave_barrier();
    }

    // ---- weights e and e (r - c), each as packed bf16 high part and the
    // bf16 rounding of the remainder: the A operands of the value MFMAs
    uint32_t phw[8], plw[8], qhw[8], qlw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float e0 = __builtin_amdgcn_exp2f(x[2 * u] - m);
      const float e1 = __builtin_amdgcn_exp2f(x[2 * u + 1] - m);
      const float f0 = e0 * (racc[2 * u] - cref);
      const float f1 = e1 * (racc[2 * u + 1] - cref);
      lsum += e0 + e1;
      bsum += f0 + f1;
      const uint32_t ph = pack_bf16(e0, e1);
      const uint32_t qh = pack_bf16(f0, f1);
      phw[u] = ph;
      qhw[u] = qh;
      plw[u] = pack_bf16(e0 - bf16_lo(ph), e1 - bf16_hi(ph));
      qlw[u] = pack_bf16(f0 - bf16_lo(qh), f1 - bf16_hi(qh));
    }

    // ---- value MFMAs over the two 16-key halves of the block
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const bf16x8 a_ph = as_bf16x8(phw[4 * uu], phw[4 * uu + 1], phw[4 * uu + 2], phw[4 * uu + 3]);
      const bf16x8 a_pl = as_bf16x8(plw[4 * uu], plw[4 * uu + 1], plw[4 * uu + 2], plw[4 * uu + 3]);
      const bf16x8 a_qh = as_bf16x8(qhw[4 * uu], qhw[4 * uu + 1], qhw[4 * uu + 2], qhw[4 * uu + 3]);
      const bf16x8 a_ql = as_bf16x8(qlw[4 * uu], qlw[4 * uu + 1], qlw[4 * uu + 2], qlw[4 * uu + 3]);
      // V rows of key slots e = 0..7: keys 16 uu + (e < 4 ? 4 half + e : 8 + 4 half + e - 4)
      uint32_t vw[8][(P::NT + 1) / 2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * uu + (e < 4 ? 4 * half + e : 8 + 4 * half + (e - 4));
        const char* vp = &kv_lds[buf][1][key * P::LSTR + col * (2 * P::NT)];
        if constexpr (P::NT == 4) {
          const i32x2 w = *reinterpret_cast<const i32x2*>(vp);
          vw[e][0] = (uint32_t)w[0];
          vw[e][1] = (uint32_t)w[1];
        } else {
          vw[e][0] = *reinterpret_cast<const uint32_t*>(vp);
        }
      }
#pragma unroll
      for (int j = 0; j < P::NT; ++j) {
        uint32_t bw[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) bw[z] = pair_halves(vw[2 * z][j >> 1], vw[2 * z + 1][j >> 1], j & 1);
        const bf16x8 vop = as_bf16x8(bw[0], bw[1], bw[2], bw[3]);
        accA[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_ph, vop, accA[j], 0, 0, 0);
        accA[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_pl, vop, accA[j], 0, 0, 0);
        accC[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_qh, vop, accC[j], 0, 0, 0);
        accC[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_ql, vop, accC[j], 0, 0, 0);
      }
    }
  };

  // Pipeline, one barrier per block: block kb is contracted from LDS buffer
  // kb % 2 while block kb + 1 goes from registers into the other buffer and
  // block kb + 3 is loaded from HBM into the registers just freed (two
  // register stages, so each load has two blocks of contraction to land).
  // One pipeline step for block kb, with `next` holding block kb + 1's pieces
  // (register stage (kb + 1) % 2, named statically by the 2-way unrolled loop).
  // Loads and stores run unconditionally: loads past the sequence are
  // range-checked to zeros without touching memory, and uniform control flow
  // lets the compiler wait only for the older register stage.
  auto step = [&](int kb, int buf, i32x4 (&next)[P::PPT]) {
    if (kb < wave_nkb) contract(kb, buf);
    store_tile(buf ^ 1, next);
    load_tile(kb + 3, next);
    __syncthreads();
  };
  load_tile(0, stage[0]);
  load_tile(1, stage[1]);
  store_tile(0, stage[0]);
  load_tile(2, stage[0]);
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, 0, stage[1]);
    step(kb + 1, 1, stage[0]);
  }

  // ---- finalise: per-row l and Bs to the output layout through LDS
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float btot = bsum + __shfl_xor(bsum, 32);
  if (half == 0) {
    row_lds[wave][0][col] = ltot;
    row_lds[wave][1][col] = btot;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int lr = 8 * (r >> 2) + 4 * half + (r & 3);  // row within the wave
    const int t = wrow0 + lr;
    if (t >= T) continue;
    float4 o = {0.f, 0.f, 0.f, 0.f};
    if (t < n) {
      const float l = row_lds[wave][0][lr];
      const float g = 1.f + row_lds[wave][1][lr] / l;
      float ov[P::NT];
#pragma unroll
      for (int j = 0; j < P::NT; ++j) ov[j] = (accA[j][r] * g - accC[j][r]) / l;
      if constexpr (P::NT == 4) {
        o = float4{ov[0], ov[1], ov[2], ov[3]};
      } else {
        o = float4{ov[0], ov[1], 0.f, 0.f};
      }
    }
    float* dst = obase + (size_t)t * D + P::NT * col;
    if constexpr (P::NT == 4) {
      *reinterpret_cast<float4*>(dst) = o;
    } else {
      *reinterpret_cast<f32x2*>(dst) = f32x2{o.x, o.y};
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int nrb = (a.T + kRows - 1) / kRows;
  dim3 grid(nrb, a.H_q, a.B);
  if (a.d == 64) {
    hipLaunchKernelGGL((prefill_kernel<64>), grid, dim3(256), 0, st,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.rho),
                       static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                       a.seq_lens, a.out, a.H_q, a.H_kv, a.G, a.T, a.S_max, a.scale * kLog2e);
  } else {
    hipLaunchKernelGGL((prefill_kernel<128>), grid, dim3(256), 0, st,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.rho),
                       static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                       a.seq_lens, a.out, a.H_q, a.H_kv, a.G, a.T, a.S_max, a.scale * kLog2e);
  }
  return hipGetLastError();
}

}  // namespace parallax
