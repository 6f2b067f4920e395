// Parallax causal prefill backward on CDNA4 (gfx950): gradients of q, rho,
// k and v for an upstream gradient dO of the output.
//
// Forward (paper page "Parallax: Parameterized Local Linear Attention for
// Language Modeling", "Abstract"; blog "Parallax: Breaking the Boundary Bias
// with Parameterized Local Linear Attention", "The Core Insight: Covariance
// Correction", output equation), row t over keys j <= t:
//
//   w_j = softmax_j(s), s_j = scale q_t.k_j, r_j = rho_t.k_j, rbar = sum w r,
//   out_t = mu_v - S_KV rho_t = sum_j w_j (1 - u_j) v_j,  u_j = r_j - rbar.
//
// Differentiating, with g_j = dO_t.v_j, G = dO_t.mu_v and Dt = dO_t.out_t:
//
//   dv_j  += w_j (1 - u_j) dO_t
//   dr_j   = w_j (G - g_j)                      -> drho_t += sum_j dr_j k_j,  dk_j += dr_j rho_t
//   ds_j   = w_j (g_j (1 - u_j) + u_j G - Dt)   -> dq_t += scale sum_j ds_j k_j,  dk_j += scale ds_j q_t
//
// Every term uses r only through u = r - rbar, so a large common offset of
// rho.k never enters; r is recomputed relative to c_t = rho_t.k_0 (the
// forward's reference, saved with the log2-sum-exp and rbar - c_t), and
// u = (r - c_t) - (rbar - c_t). The weights are recomputed from the saved
// log2-sum-exp, so no T x T matrix is stored.
//
// Two launches:
//  1. dq/drho: per 128 query rows (8 waves x 16 rows), over key blocks of 32
//     staged in LDS (as the forward). Each lane first splits its row's dO
//     (fp32) into bf16 high and low parts and forms the row's G and Dt (from
//     the saved mu_v and the output), and leaves both in the workspace for
//     the second launch. s, r - c and g come from v_mfma_f32_16x16x32_bf16
//     in the forward's transposed layout; ds and dr (fp32, split into bf16
//     high and low parts) contract with K, whose operand the transposing LDS
//     load reads straight from the row-major tile.
//  2. dk/dv: per 128 keys (8 waves x 16 keys) of one KV head, over the
//     query-row blocks of 32 of every head of its group that see those keys,
//     with q, rho, dO (high, low) and the row statistics staged in LDS.
//     s, r - c, g come out with keys as columns, so each lane holds one key
//     and 8 rows: exactly the A-operand slots of P^T dO, ds^T q and dr^T rho,
//     whose B operands the transposing load reads from the staged tiles.
// Products with fp32 weights use the bf16 high part and the bf16 rounding of
// the remainder of the weight (and of dO), so the contractions keep about
// 2^-16 relative accuracy. Each key block and row block is paired with its
// mirror so every workgroup carries the same causal work.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 512;  // 8 waves
constexpr int kQRows = 128;    // dq kernel: query rows per workgroup
constexpr int kQKeys = 32;     // dq kernel: keys per staged block
constexpr int kKKeys = 128;    // dkv kernel: keys per workgroup
constexpr int kKRows = 32;     // dkv kernel: query rows per staged block

template <int D>
struct Bw {
  static constexpr int ROWB = D * 2;          // bytes per bf16 row
  static constexpr int STR = ROWB + 32;       // LDS row stride (bytes)
  static constexpr int KST = D / 32;          // k-steps of a d-contraction
  static constexpr int DPL = D / 16;          // N-tiles over d
  static constexpr int TILE = 32 * STR;       // one staged 32-row bf16 tile
  static constexpr int PIECES = 32 * ROWB / 16;  // 16-byte pieces per tile
};

// B operand of N-tile j (dims 16 j .. 16 j + 15) for key/row slots
// e = 0..7 (tile row 16 (e / 4) + 4 g + e % 4) from a row-major 32-row tile:
// two transposing loads; within each group of 16 lanes, lane 4 a + b receives
// element b of the 8-byte pieces addressed by lanes a, a + 4, a + 8, a + 12.
template <int STR>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int g, int c, int j) {
  const char* p = tile + (4 * g + (c >> 2)) * STR + 32 * j + 8 * (c & 3);
  const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * STR));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 8 fp32 values as bf16 high parts and bf16 roundings of the remainders.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t ph = pack_bf16(x[2 * u], x[2 * u + 1]);
    h[u] = ph;
    l[u] = pack_bf16(x[2 * u] - bf16_lo(ph), x[2 * u + 1] - bf16_hi(ph));
  }
  hi = as_bf16x8(h[0], h[1], h[2], h[3]);
  lo = as_bf16x8(l[0], l[1], l[2], l[3]);
}

// As split8, also adding to `sum` the values the two parts represent.
__device__ __forceinline__ void split8_sum(const float (&x)[8], bf16x8& hi, bf16x8& lo, float& sum) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t ph = pack_bf16(x[2 * u], x[2 * u + 1]);
    h[u] = ph;
    const uint32_t pl = pack_bf16(x[2 * u] - bf16_lo(ph), x[2 * u + 1] - bf16_hi(ph));
    l[u] = pl;
    sum += (bf16_lo(ph) + bf16_lo(pl)) + (bf16_hi(ph) + bf16_hi(pl));
  }
  hi = as_bf16x8(h[0], h[1], h[2], h[3]);
  lo = as_bf16x8(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroups are dealt to the 8 XCDs in linear order; this remaps the
// linear index so that each XCD takes a contiguous range of (x, y, z) tiles
// (x fastest), whose neighbours share their K/V or q/rho/dO rows in that
// XCD's L2. Returns the remapped x, y, z.
__device__ __forceinline__ void xcd_tile(int& x, int& y, int& z) {
  x = blockIdx.x;
  y = blockIdx.y;
  z = blockIdx.z;
  const unsigned long long total = (unsigned long long)gridDim.x * gridDim.y * gridDim.z;
  if (total < (1ull << 31) && total % 8u == 0u) {
    const unsigned tot = (unsigned)total;
    const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned L = (lin % 8u) * (tot / 8u) + lin / 8u;
    x = (int)(L % gridDim.x);
    y = (int)((L / gridDim.x) % gridDim.y);
    z = (int)(L / (gridDim.x * gridDim.y));
  }
}

__device__ __forceinline__ bf16x8 load8(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(p));
}

// ---------------------------------------------------------------------------
// 1. dq, drho: one row block (128 rows from rb * 128) of one (b, h).
template <int D>
__device__ __forceinline__ void dq_rows(const BwdArgs& a, int rb, int h, int b,
                                        char (&lds)[2][2][Bw<D>::TILE]) {
  using P = Bw<D>;
  const int hk = h / a.G;
  const int T = a.T;
  const int n = min(max(a.seq_lens[b], 0), T);
  const int R0 = rb * kQRows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int wrow0 = R0 + 16 * wave;
  const int my_row = wrow0 + c;
  const size_t qbase = ((size_t)b * a.H_q + h) * (size_t)T;  // row index base
  float* dq = a.dq + qbase * D;
  float* dr = a.drho + qbase * D;

  if (R0 >= n) {
    for (int i = tid; i < kQRows * D / 4; i += kThreads) {
      const int r = R0 + i / (D / 4);
      if (r < T) {
        reinterpret_cast<float4*>(dq + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<float4*>(dr + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }

  // Row operands (B of the transposed products): row my_row, dims 32 kk + 8 g.
  // dO comes in fp32 and is split here into its bf16 high and low parts; the
  // row's G = dO.mu_v and Dt = dO.out are summed over this lane's dims and
  // the row's 4 lanes (g). The parts and (G, Dt) also go to the workspace,
  // where the dk/dv launch that follows reads them (rows below n only; every
  // such row belongs to exactly one workgroup of this launch).
  const bool live = my_row < n;
  const size_t roff = (qbase + (live ? my_row : 0)) * D + 8 * g;
  bf16x8 qop[P::KST], rop[P::KST], dhop[P::KST], dlop[P::KST];
  float Gr = 0.f, Dr = 0.f;
#pragma unroll
  for (int kk = 0; kk < P::KST; ++kk) {
    const bf16x8 z = __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0});
    qop[kk] = live ? load8(reinterpret_cast<const char*>(
                         static_cast<const __bf16*>(a.q) + roff + 32 * kk)) : z;
    rop[kk] = live ? load8(reinterpret_cast<const char*>(
                         static_cast<const __bf16*>(a.rho) + roff + 32 * kk)) : z;
    float x[8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const size_t o4 = roff + 32 * kk + 4 * h2;
      const float4 dv4 = live ? *reinterpret_cast<const float4*>(a.dout + o4) : float4{0.f, 0.f, 0.f, 0.f};
      const float4 m4 = live ? *reinterpret_cast<const float4*>(a.mu + o4) : float4{0.f, 0.f, 0.f, 0.f};
      const float4 o44 = live ? *reinterpret_cast<const float4*>(a.out + o4) : float4{0.f, 0.f, 0.f, 0.f};
      x[4 * h2 + 0] = dv4.x;
      x[4 * h2 + 1] = dv4.y;
      x[4 * h2 + 2] = dv4.z;
      x[4 * h2 + 3] = dv4.w;
      Gr += dv4.x * m4.x + dv4.y * m4.y + dv4.z * m4.z + dv4.w * m4.w;
      Dr += dv4.x * o44.x + dv4.y * o44.y + dv4.z * o44.z + dv4.w * o44.w;
    }
    split8(x, dhop[kk], dlop[kk]);
    if (live) {
      *reinterpret_cast<bf16x8*>(a.dhi + roff + 32 * kk) = dhop[kk];
      *reinterpret_cast<bf16x8*>(a.dlo + roff + 32 * kk) = dlop[kk];
    }
  }
  // the row's 4 lanes are c, c + 16, c + 32, c + 48
  Gr += __shfl_xor(Gr, 16);
  Dr += __shfl_xor(Dr, 16);
  Gr += __shfl_xor(Gr, 32);
  Dr += __shfl_xor(Dr, 32);
  if (live && g == 0) a.gd[qbase + my_row] = float2{Gr, Dr};
  float lse2 = 0.f, crow = 0.f, rbc = 0.f;
  if (live) {
    const float4 st = a.stats[qbase + my_row];
    lse2 = st.x;
    crow = st.y;
    rbc = st.z;
  }
  const f32x4 rinit = {-crow, -crow, -crow, -crow};

  const size_t kvslice = ((size_t)b * a.H_kv + hk) * (size_t)a.S_max * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const __bf16*>(a.k) + kvslice, (uint32_t)n * P::ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const __bf16*>(a.v) + kvslice, (uint32_t)n * P::ROWB);
  const int nkb = (min(R0 + kQRows, n) + kQKeys - 1) / kQKeys;
  const int wave_nkb = wrow0 < n ? min(wrow0 + 15, n - 1) / kQKeys + 1 : 0;

  // K and V pieces: PIECES per tile, 2 tiles, kThreads threads.
  constexpr int PPT = 2 * P::PIECES / kThreads;
  auto piece = [&](int i, int& which, int& idx) {
    if constexpr (PPT >= 2) {
      which = i < PPT / 2 ? 0 : 1;
      idx = tid + kThreads * (i % (PPT / 2));
    } else {
      which = __builtin_amdgcn_readfirstlane(tid / (kThreads / 2));
      idx = tid % (kThreads / 2);
    }
  };
  i32x4 stage[2][PPT];
  auto load_tile = [&](int kb, i32x4 (&dst)[PPT]) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      int which, idx;
      piece(i, which, idx);
      const uint32_t off = (uint32_t)(kb * kQKeys + idx / (P::ROWB / 16)) * P::ROWB + (idx % (P::ROWB / 16)) * 16;
      dst[i] = __builtin_amdgcn_raw_buffer_load_b128(which ? vrs : krs, off, 0, 0);
    }
  };
  auto store_tile = [&](int buf, const i32x4 (&src)[PPT]) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      int which, idx;
      piece(i, which, idx);
      *reinterpret_cast<i32x4*>(&lds[buf][which][(idx / (P::ROWB / 16)) * P::STR + (idx % (P::ROWB / 16)) * 16]) = src[i];
    }
  };

  f32x4 accQ[P::DPL], accR[P::DPL];
#pragma unroll
  for (int j = 0; j < P::DPL; ++j) {
    accQ[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accR[j] = accQ[j];
  }
  // This lane's share of sum_j ds_j and sum_j dr_j for row my_row, as the
  // MFMAs see them. Both sums vanish exactly (softmax gradients sum to zero;
  // sum_j w_j (G - g_j) = G - dO.mu_v = 0), so dq = scale sum_j ds_j k_j equals
  // scale sum_j ds_j (k_j - k_0); forming it that way cancels the rounding of
  // those identities against the key offset (and makes row 0, which sees only
  // k_0, exactly zero).
  float sum_ds = 0.f, sum_dr = 0.f;

  auto contract = [&](int kb, int buf) {
    // s, r - c, g for row my_row (lane column c), keys 16 T + 4 g + i
    f32x4 sc[2], rr[2], gg[2];
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2) {
      sc[T2] = f32x4{0.f, 0.f, 0.f, 0.f};
      gg[T2] = sc[T2];
      rr[T2] = rinit;
      const char* krow = &lds[buf][0][(16 * T2 + c) * P::STR + 16 * g];
      const char* vrow = &lds[buf][1][(16 * T2 + c) * P::STR + 16 * g];
#pragma unroll
      for (int kk = 0; kk < P::KST; ++kk) {
        const bf16x8 kop = load8(krow + 64 * kk);
        const bf16x8 vop = load8(vrow + 64 * kk);
        sc[T2] = mfma(kop, qop[kk], sc[T2]);
        rr[T2] = mfma(kop, rop[kk], rr[T2]);
        gg[T2] = mfma(vop, dhop[kk], gg[T2]);
        gg[T2] = mfma(vop, dlop[kk], gg[T2]);
      }
    }
    float dsv[8], drv[8];
    const bool diag = kb * kQKeys + kQKeys - 1 > wrow0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = sc[e >> 2][e & 3];
      float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s, a.scale_log2, -lse2));
      if (diag) {
        const int key = kb * kQKeys + 16 * (e >> 2) + 4 * g + (e & 3);
        w = key <= my_row ? w : 0.f;
      }
      const float u = rr[e >> 2][e & 3] - rbc;
      const float gv = gg[e >> 2][e & 3];
      drv[e] = w * (Gr - gv);
      dsv[e] = w * (gv * (1.f - u) + u * Gr - Dr);
    }
    bf16x8 ds_h, ds_l, dr_h, dr_l;
    split8_sum(dsv, ds_h, ds_l, sum_ds);
    split8_sum(drv, dr_h, dr_l, sum_dr);
    const char* ktile = &lds[buf][0][0];
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      const bf16x8 kb_op = tr_operand<P::STR>(ktile, g, c, j);
      accQ[j] = mfma(ds_h, kb_op, accQ[j]);
      accQ[j] = mfma(ds_l, kb_op, accQ[j]);
      accR[j] = mfma(dr_h, kb_op, accR[j]);
      accR[j] = mfma(dr_l, kb_op, accR[j]);
    }
  };

  auto step = [&](int kb, int buf, i32x4 (&next)[PPT]) {
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

  // row sums over the four lane groups holding a row's keys
  sum_ds += __shfl_xor(sum_ds, 16);
  sum_ds += __shfl_xor(sum_ds, 32);
  sum_dr += __shfl_xor(sum_dr, 16);
  sum_dr += __shfl_xor(sum_dr, 32);
  float k0[P::DPL];  // key 0 at dims 16 j + c
#pragma unroll
  for (int j = 0; j < P::DPL; ++j)
    k0[j] = (float)static_cast<const __bf16*>(a.k)[kvslice + 16 * j + c];
  // accumulator element i of lane (g, c): row 4 g + i of the wave, dim 16 j + c
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sq = __shfl(sum_ds, 4 * g + i);
    const float sr = __shfl(sum_dr, 4 * g + i);
    const int t = wrow0 + 4 * g + i;
    if (t >= T) continue;
    const bool tl = t < n;
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      dq[(size_t)t * D + 16 * j + c] = tl ? a.scale * (accQ[j][i] - sq * k0[j]) : 0.f;
      dr[(size_t)t * D + 16 * j + c] = tl ? accR[j][i] - sr * k0[j] : 0.f;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][Bw<D>::TILE];  // [buffer][K, V]
  const int nrb = (a.T + kQRows - 1) / kQRows;
  int x, h, b;
  xcd_tile(x, h, b);
  dq_rows<D>(a, nrb - 1 - x, h, b, lds);
  if (x != nrb - 1 - x) {
    __syncthreads();
    dq_rows<D>(a, x, h, b, lds);
  }
}

// ---------------------------------------------------------------------------
// 2. dk, dv: one key block (128 keys from kb * 128) of one (b, KV head).
struct RowStat {
  float lse2, c, rbc, G, Dt, pad0, pad1, pad2;
};

template <int D>
__device__ __forceinline__ void dkv_keys(const BwdArgs& a, int kb, int hk, int b,
                                         char (&lds)[4][4][Bw<D>::TILE], RowStat (&rst)[4][kKRows]) {
  using P = Bw<D>;
  const int G = a.G;
  const int T = a.T;
  const int n = min(max(a.seq_lens[b], 0), T);
  const int J0 = kb * kKKeys;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int kw0 = J0 + 16 * wave;  // this wave's first key
  const size_t kvslice = ((size_t)b * a.H_kv + hk) * (size_t)a.S_max;  // row index base
  float* dk = a.dk + kvslice * D;
  float* dv = a.dv + kvslice * D;

  if (J0 >= n) {  // keys past the sequence (up to S_max): zero gradients
    for (int i = tid; i < kKKeys * D / 4; i += kThreads) {
      const int r = J0 + i / (D / 4);
      if (r < a.S_max) {
        reinterpret_cast<float4*>(dk + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<float4*>(dv + (size_t)r * D)[i % (D / 4)] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }

  // Key operands (B of the row-major products): key kw0 + c, dims 32 kk + 8 g.
  const int my_key = kw0 + c;
  const bool klive = my_key < n;
  bf16x8 kop[P::KST], vop[P::KST];
  {
    const size_t off = (kvslice + (klive ? my_key : 0)) * D + 8 * g;
    const bf16x8 z = __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0});
#pragma unroll
    for (int kk = 0; kk < P::KST; ++kk) {
      kop[kk] = klive ? load8(reinterpret_cast<const char*>(static_cast<const __bf16*>(a.k) + off + 32 * kk)) : z;
      vop[kk] = klive ? load8(reinterpret_cast<const char*>(static_cast<const __bf16*>(a.v) + off + 32 * kk)) : z;
    }
  }

  // Steps: every head of the group, row blocks from the one holding key J0
  // to the last one holding a row < n.
  const int rb0 = J0 / kKRows;
  const int nrb = (n - 1) / kKRows - rb0 + 1;
  const int S = G * nrb;

  // Staged pieces: tiles q, rho, dO high, dO low (PIECES each) plus one
  // 32-byte row record (16 bytes of stats + 8 of (G, Dt)) per row.
  constexpr int PPT = 4 * P::PIECES / kThreads;
  struct Stage {
    i32x4 p[PPT];
    float4 st;
    float2 gd;
  };
  auto src = [&](int s, int tile, int rb2, __amdgpu_buffer_rsrc_t& rs) {
    (void)rb2;
    const int hh = s < S ? s / nrb : 0;
    const int h = hk * G + hh;
    const size_t base = ((size_t)b * a.H_q + h) * (size_t)T * D;
    const void* ptr = tile == 0 ? (const void*)(static_cast<const __bf16*>(a.q) + base)
                    : tile == 1 ? (const void*)(static_cast<const __bf16*>(a.rho) + base)
                    : tile == 2 ? (const void*)(a.dhi + base)
                                : (const void*)(a.dlo + base);
    rs = make_rsrc(ptr, s < S ? (uint32_t)n * P::ROWB : 0u);
  };
  auto load = [&](int s, Stage& st) {
    const int rb2 = rb0 + (s < S ? s % nrb : 0);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      int tile, idx;
      if constexpr (PPT >= 4) {
        tile = i / (PPT / 4);
        idx = tid + kThreads * (i % (PPT / 4));
      } else {
        const int p = tid + kThreads * i;
        tile = __builtin_amdgcn_readfirstlane(p / P::PIECES);
        idx = p % P::PIECES;
      }
      __amdgpu_buffer_rsrc_t rs;
      src(s, tile, rb2, rs);
      const uint32_t off = (uint32_t)(rb2 * kKRows + idx / (P::ROWB / 16)) * P::ROWB + (idx % (P::ROWB / 16)) * 16;
      st.p[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
    const int hh = s < S ? s / nrb : 0;
    const size_t rbase = ((size_t)b * a.H_q + hk * G + hh) * (size_t)T;
    const uint32_t nb = s < S ? (uint32_t)n : 0u;
    const uint32_t row = (uint32_t)(rb2 * kKRows + (tid & (kKRows - 1)));
    const i32x4 s4 = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(a.stats + rbase, nb * 16), row * 16, 0, 0);
    const i32x2 g2 = __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(a.gd + rbase, nb * 8), row * 8, 0, 0);
    st.st = __builtin_bit_cast(float4, s4);
    st.gd = __builtin_bit_cast(float2, g2);
  };
  auto store = [&](int buf, const Stage& st) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      int tile, idx;
      if constexpr (PPT >= 4) {
        tile = i / (PPT / 4);
        idx = tid + kThreads * (i % (PPT / 4));
      } else {
        const int p = tid + kThreads * i;
        tile = __builtin_amdgcn_readfirstlane(p / P::PIECES);
        idx = p % P::PIECES;
      }
      *reinterpret_cast<i32x4*>(&lds[buf][tile][(idx / (P::ROWB / 16)) * P::STR + (idx % (P::ROWB / 16)) * 16]) = st.p[i];
    }
    if (tid < kKRows)
      rst[buf][tid] = RowStat{st.st.x, st.st.y, st.st.z, st.gd.x, st.gd.y, 0.f, 0.f, 0.f};
  };

  f32x4 accK[P::DPL], accV[P::DPL];
#pragma unroll
  for (int j = 0; j < P::DPL; ++j) {
    accK[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accV[j] = accK[j];
  }

  auto contract = [&](int s, int buf) {
    const int rb2 = rb0 + s % nrb;
    const int r0 = rb2 * kKRows;  // first row of the block
    if (r0 + kKRows - 1 < kw0) return;  // every row of the block precedes this wave's keys
    // s, r - c, g with rows 16 T + 4 g + i (block-local) down, key c across
    f32x4 sc[2], rr[2], gg[2];
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2) {
      sc[T2] = f32x4{0.f, 0.f, 0.f, 0.f};
      gg[T2] = sc[T2];
#pragma unroll
      for (int i = 0; i < 4; ++i) rr[T2][i] = -rst[buf][16 * T2 + 4 * g + i].c;
      const int roff = (16 * T2 + c) * P::STR + 16 * g;
      // Every row read of a pair of tiles (q and rho, then dO high and low)
      // is issued before the MFMAs that use them (order pinned).
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 x0[P::KST], x1[P::KST];
#pragma unroll
        for (int kk = 0; kk < P::KST; ++kk) {
          x0[kk] = load8(&lds[buf][2 * half][roff + 64 * kk]);
          x1[kk] = load8(&lds[buf][2 * half + 1][roff + 64 * kk]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < P::KST; ++kk) {
          if (half == 0) {
            sc[T2] = mfma(x0[kk], kop[kk], sc[T2]);
            rr[T2] = mfma(x1[kk], kop[kk], rr[T2]);
          } else {
            gg[T2] = mfma(x0[kk], vop[kk], gg[T2]);
            gg[T2] = mfma(x1[kk], vop[kk], gg[T2]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float pv[8], dsv[8], drv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int rl = 16 * (e >> 2) + 4 * g + (e & 3);
      const RowStat rs = rst[buf][rl];
      const int t = r0 + rl;
      const bool ok = t >= my_key && t < n;
      const float w = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e >> 2][e & 3], a.scale_log2, -rs.lse2)) : 0.f;
      const float u = rr[e >> 2][e & 3] - rs.rbc;
      const float gv = gg[e >> 2][e & 3];
      pv[e] = w * (1.f - u);
      drv[e] = w * (rs.G - gv);
      dsv[e] = a.scale * w * (gv * (1.f - u) + u * rs.G - rs.Dt);
    }
    bf16x8 p_h, p_l, ds_h, ds_l, dr_h, dr_l;
    split8(pv, p_h, p_l);
    split8(dsv, ds_h, ds_l);
    split8(drv, dr_h, dr_l);
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      const bf16x8 oh = tr_operand<P::STR>(&lds[buf][2][0], g, c, j);
      const bf16x8 ol = tr_operand<P::STR>(&lds[buf][3][0], g, c, j);
      accV[j] = mfma(p_h, oh, accV[j]);
      accV[j] = mfma(p_l, oh, accV[j]);
      accV[j] = mfma(p_h, ol, accV[j]);
      const bf16x8 qo = tr_operand<P::STR>(&lds[buf][0][0], g, c, j);
      const bf16x8 ro = tr_operand<P::STR>(&lds[buf][1][0], g, c, j);
      accK[j] = mfma(ds_h, qo, accK[j]);
      accK[j] = mfma(ds_l, qo, accK[j]);
      accK[j] = mfma(dr_h, ro, accK[j]);
      accK[j] = mfma(dr_l, ro, accK[j]);
    }
  };

  // Two row blocks per barrier: blocks s, s + 1 are contracted from LDS
  // buffers pb, pb + 1 while blocks s + 2, s + 3 go from registers into the
  // other pair and blocks s + 4, s + 5 are loaded (a pair of steps of
  // contraction covers each load). Against one block per barrier this halves
  // the barriers and the operand waits after them: the backward step took
  // 2625-2709 us against 2684-2730 us. It needs 256 registers (no spills)
  // and 148 KB of LDS.
  Stage st0, st1;
  auto groupstep = [&](int s, int pb) {
    if (s < S) contract(s, pb);
    if (s + 1 < S) contract(s + 1, pb + 1);
    store(pb ^ 2, st0);
    store((pb ^ 2) + 1, st1);
    load(s + 4, st0);
    load(s + 5, st1);
    __syncthreads();
  };
  load(0, st0);
  load(1, st1);
  store(0, st0);
  store(1, st1);
  load(2, st0);
  load(3, st1);
  __syncthreads();
  for (int s = 0; s < S; s += 4) {
    groupstep(s, 0);
    if (s + 2 < S) groupstep(s + 2, 2);
  }

  // accumulator element i of lane (g, c): key kw0 + 4 g + i, dim 16 j + c
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kw0 + 4 * g + i;
    if (key >= a.S_max) continue;
    const bool kl = key < n;
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      dk[(size_t)key * D + 16 * j + c] = kl ? accK[j][i] : 0.f;
      dv[(size_t)key * D + 16 * j + c] = kl ? accV[j][i] : 0.f;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[4][4][Bw<D>::TILE];  // [buffer][q, rho, dO hi, dO lo]
  __shared__ RowStat rst[4][kKRows];
  const int nkb = (a.S_max + kKKeys - 1) / kKKeys;
  int x, hk, b;
  xcd_tile(x, hk, b);
  dkv_keys<D>(a, x, hk, b, lds, rst);  // early (heavy) key block
  if (x != nkb - 1 - x) {
    __syncthreads();
    dkv_keys<D>(a, nkb - 1 - x, hk, b, lds, rst);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  const int nrb = (a.T + kQRows - 1) / kQRows;
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((nrb + 1) / 2, a.H_q, a.B), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.S_max + kKKeys - 1) / kKKeys;
  hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3((nkb + 1) / 2, a.H_kv, a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_backward(const BwdArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_bwd_d<64>(a, st) : launch_bwd_d<128>(a, st);
}

}  // namespace parallax
