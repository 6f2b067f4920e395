// Parallax decode on CDNA4 (gfx950): split-KV partial kernel and combine kernel.
//
// What is computed (paper page "Parallax: Parameterized Local Linear Attention
// for Language Modeling", "Abstract"; blog "Parallax: Breaking the Boundary
// Bias with Parameterized Local Linear Attention", "The Core Insight:
// Covariance Correction", output equation; "Hardware Efficiency": softmax
// and covariance branches fused into one pass over the KV stream):
//
//   out = mu_v - S_KV rho,  S_KV = sum_i w_i (v_i - mu_v)(k_i - mu_k)^T.
//
// Applying S_KV to rho key by key gives a streaming form. With
// r_i = rho . k_i, e_i = exp(s_i - m), l = sum e_i, A = sum e_i v_i,
// Bs = sum e_i r_i and C = sum e_i r_i v_i:
//
//   S_KV rho = sum_i w_i r_i v_i - (rho . mu_k) mu_v = C/l - (Bs/l)(A/l)
//   out      = (A (1 + Bs/l) - C) / l.
//
// Replacing r_i by r_i - c for any constant c leaves `out` unchanged
// (Bs -> Bs - c l, C -> C - c A), so each wave accumulates r relative to the
// r of the first key it sees; this removes any large common offset of
// rho . k before it can cancel. Partial states with different max (m) and
// reference (c) merge exactly: rescale by exp(m_j - M) and shift by
// (c_j - c) as above, an associative and commutative merge.
//
// Work layout. A workgroup of 4 waves (8 for bf16 at d = 64) owns one (b,
// KV head, group of <= 4 query heads, or <= 8 when the KV head has more
// than 4, key range of `chunk` keys). Each wave takes every 4th (8th) block
// of 32 keys. Per block a lane loads its K and V pieces from HBM into
// registers with range-checked buffer loads (rows at or past the sequence
// length come back as zeros, so padding is never read). Both are read in
// whole rows per instruction and carry the non-temporal streaming hint. V
// needs no rearranging; for bf16 the wave passes its K block through a
// private LDS region to form the score MFMA's operand (16 rows x 64 bytes per
// MFMA). Loading that operand straight from HBM fetched half of each 128-byte
// line per instruction and could not take the hint: 2-5% slower. Two MFMA
// contractions do the arithmetic:
//   scores:  [32 keys x d] x [d x 16 probe columns] with v_mfma_f32_16x16x32_bf16,
//            probe column 4h+t holds q_h for t in {0,1} and rho_h for t in {2,3},
//            so one pass gives s and r for all (up to 4) heads of the group;
//   values:  [16 rows x 32 keys] x [32 keys x d], rows 4h+t holding, for head h,
//            e (t=0,1) or e*(r-c) (t=2,3) split into a bf16 high part (t even)
//            and the bf16 rounding of the remainder (t odd), so the fp32
//            weights survive the bf16 contraction to about 2^-17.
// The score accumulator layout of the MFMA puts, in lane (g = lane/16,
// c = lane%16), the values of probe column c for keys 16T + 4g + i
// (T = 0, 1; i = 0..3): exactly the 8 key slots that lane must supply as the
// A operand of the value MFMA, so no data moves between lanes except one DPP
// quad permute that hands s to the lanes holding r. V needs no transpose: the
// lane loads 8 rows x (d/16) contiguous elements and hands element j of each
// row to N-tile j (value column c of tile j is dimension (d/16) c + j).
// fp32 inputs are split into bf16 high and low parts and contracted as
// hi*hi + hi*lo + lo*hi (scores) and P*(v_hi + v_lo) (values).
// The softmax max is rescaled lazily: only when a block's max exceeds the
// running reference by more than 2^8, which keeps every exp below 256.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace parallax {

namespace {

constexpr int kBlockKeys = 32;

// Waves per workgroup, by the bytes of one K or V row. With 128-byte rows
// (bf16 at d = 64) eight waves keep as many bytes in flight per compute unit
// as four do with 256-byte rows (bf16 at d = 128, fp32 at d = 64), with one
// workgroup per compute unit (gqa shape at d = 64: 4 splits of 8 waves 15.7
// us, against 16.0 for 8 splits of 4 waves, two workgroups per compute unit,
// and 16.1 for 4 splits of 4 waves). With 256-byte rows eight waves measured
// slower (4 heads per workgroup: 24.5 against 24.1 us; 8 heads: 25.65
// against 25.52).
constexpr int decode_waves(int row_bytes) { return row_bytes <= 128 ? 8 : 4; }
constexpr float kRescaleLog2 = 8.0f;

template <typename T, int D>
struct Dec {
  static constexpr int ESZ = sizeof(T);
  static constexpr int ROWB = D * ESZ;                  // bytes per K/V row
  static constexpr int KSTEPS = D / 32;                 // score MFMA k-steps
  static constexpr int DPL = D / 16;                    // value dims per lane = N-tiles
  static constexpr int KW = 8 * ESZ / 4;                // words per K piece (8 elements)
  static constexpr int VW = DPL * ESZ / 4;              // words per V row piece
  static constexpr bool F32 = (ESZ == 4);
  static constexpr int REC = 2 * D + 4;                 // fp32 words per partial record
  static constexpr int RP = ROWB / 16;                  // 16-byte pieces per K/V row
  static constexpr int KSTR = ROWB + 16;                // LDS row stride of a staged K block (bf16)
  static constexpr int KLDS = F32 ? 16 : kBlockKeys * KSTR;  // bytes of one wave's K block
};

// 8 consecutive elements (one MFMA operand) from words; fp32 gives hi and lo.
template <typename T>
__device__ __forceinline__ void to_operand(const uint32_t* w, bf16x8& hi, bf16x8& lo) {
  if constexpr (sizeof(T) == 2) {
    hi = as_bf16x8(w[0], w[1], w[2], w[3]);
  } else {
    float x[8], r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = __uint_as_float(w[i]);
      r[i] = x[i] - bf16_round(x[i]);
    }
    hi = as_bf16x8(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                   pack_bf16(x[6], x[7]));
    lo = as_bf16x8(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]), pack_bf16(r[4], r[5]),
                   pack_bf16(r[6], r[7]));
  }
}

template <typename T>
__device__ __forceinline__ uint32_t load_probe_words(const T* p, int n, uint32_t* w) {
  // 8 elements at p (16-byte aligned); n words
  const uint4* src = reinterpret_cast<const uint4*>(p);
  uint4 a = src[0];
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  if (n == 8) {
    uint4 b = src[1];
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  return 0;
}

// Cache-policy operand of a buffer access that goes to the device-coherent
// level (gfx950 "sc1"): records exchanged between the workgroups of one
// launch, which may run on different XCDs, each with its own L2.
constexpr int kCoherent = 16;

// V consecutive floats (V = 1, 2, 4) as one value.
template <int V> struct Vec;
template <> struct Vec<1> { typedef float T; };
template <> struct Vec<2> { typedef f32x2 T; };
template <> struct Vec<4> { typedef f32x4 T; };

// Record accesses at byte offset `off` of a workgroup's record range, which
// starts at `base` and is also reached through the descriptor `r`. Four
// floats move as one 16-byte buffer access (COH: at the device-coherent
// level); one or two floats as global accesses (COH: agent-scope atomics,
// also at the coherent level), which measured slightly faster than the
// narrow buffer forms in the 4-head kernel.
template <int V, bool COH>
__device__ __forceinline__ typename Vec<V>::T rec_load(const float* base, __amdgpu_buffer_rsrc_t r,
                                                       uint32_t off) {
  if constexpr (V == 4) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, COH ? kCoherent : 0));
  } else if constexpr (V == 2) {
    const uint64_t* p = reinterpret_cast<const uint64_t*>(base + off / 4);
    if constexpr (COH)
      return __builtin_bit_cast(f32x2, __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    else
      return __builtin_bit_cast(f32x2, *p);
  } else {
    const float* p = base + off / 4;
    if constexpr (COH)
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      return *p;
  }
}

template <int V, bool COH>
__device__ __forceinline__ void rec_store(typename Vec<V>::T x, float* base, __amdgpu_buffer_rsrc_t r,
                                          uint32_t off) {
  if constexpr (V == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, off, 0, COH ? kCoherent : 0);
  } else if constexpr (V == 2) {
    uint64_t* p = reinterpret_cast<uint64_t*>(base + off / 4);
    if constexpr (COH)
      __hip_atomic_store(p, __builtin_bit_cast(uint64_t, x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = __builtin_bit_cast(uint64_t, x);
  } else {
    float* p = base + off / 4;
    if constexpr (COH)
      __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = x;
  }
}

// The 16-byte record header (m, l, Bs, c): one 16-byte buffer access (COH:
// at the device-coherent level) whatever V is. Against four single-float
// accesses it saved 0.06-0.09 us per launch on gqa-decode, its d = 64 form
// and single-head, and 0.8 us on long-context (A/B, same process).
template <bool COH>
__device__ __forceinline__ f32x4 hdr_load(const float* base, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  return rec_load<4, COH>(base, r, off);
}

template <bool COH>
__device__ __forceinline__ void hdr_store(f32x4 x, float* base, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  rec_store<4, COH>(x, base, r, off);
}

// Merges the partial records of splits 0..nsv-1 of one (b, h_q) at the V
// dimensions V q .. V q + V - 1 and returns the finalised outputs. Records
// are REC = 2D+4 floats apart from byte offset `off0` of the descriptor `r`:
// (m, l, Bs, c) as one 16-byte header, then A[D] and C[D]. Online over the
// splits (the running max only grows; records with l = 0 hold no key and are
// skipped; the probe reference is the first non-empty record's), with the
// loads of NB splits issued before any of them is used. COH reads at the
// device-coherent level (records written in the same launch).
template <int D, int V, bool COH, int NB>
__device__ __forceinline__ typename Vec<V>::T merge_records(const float* base,
                                                            __amdgpu_buffer_rsrc_t r, uint32_t off0,
                                                            int nsv, int q) {
  using VT = typename Vec<V>::T;
  constexpr uint32_t RECB = (2 * D + 4) * 4;
  if (nsv <= 0) return VT{};
  float c0 = 0.f;
  bool have = false;  // the reference c0 is the first non-empty record's
  float M = -INFINITY, l = 0.f, bs = 0.f;
  VT A{}, C{};
  for (int s0 = 0; s0 < nsv; s0 += NB) {
    f32x4 hd[NB];
    VT Aw[NB], Cw[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t rec = off0 + (uint32_t)min(s0 + i, nsv - 1) * RECB;
      hd[i] = hdr_load<COH>(base, r, rec);
      Aw[i] = rec_load<V, COH>(base, r, rec + 16 + 4 * V * q);
      Cw[i] = rec_load<V, COH>(base, r, rec + 16 + 4 * D + 4 * V * q);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float ms = hd[i][0], lw = hd[i][1], bw = hd[i][2], cw = hd[i][3];
      if (s0 + i < nsv && lw > 0.f) {  // a record with l = 0 holds no key
        if (!have) {
          c0 = cw;
          have = true;
        }
        if (ms > M) {
          const float f = exp2f(M - ms);
          l *= f;
          bs *= f;
          A *= f;
          C *= f;
          M = ms;
        }
        const float al = exp2f(ms - M);
        const float sh = cw - c0;
        l += al * lw;
        bs += al * (bw + sh * lw);
        A += al * Aw[i];
        C += al * (Cw[i] + sh * Aw[i]);
      }
    }
  }
  if (!(l > 0.f)) return VT{};
  const float gn = 1.f + bs / l;
  return (A * gn - C) / l;
}

// merge_records with at most 8 record loads in flight, and no more than there
// are records: a batch's loads past the last record repeat it, and in the
// merging workgroup's tail those repeats cost time (at 4 splits, 0.2 us of
// gqa-decode and 0.5 us at 8 query heads per KV head).
template <int D, int V, bool COH>
__device__ __forceinline__ typename Vec<V>::T merge_splits(const float* base,
                                                           __amdgpu_buffer_rsrc_t r, uint32_t off0,
                                                           int nsv, int q) {
  if (nsv <= 2) return merge_records<D, V, COH, 2>(base, r, off0, nsv, q);
  if (nsv <= 4) return merge_records<D, V, COH, 4>(base, r, off0, nsv, q);
  return merge_records<D, V, COH, 8>(base, r, off0, nsv, q);
}

// MT (several new tokens per sequence): every (query head, token) pair is a
// query of its own ("virtual head" v = h * ntok + t, so q, rho and out keep
// their [B, H_q, ntok, d] layout and H_q, G count virtual heads), seq_lens
// holds the chunk lengths and past_lens the cached lengths, and token t of a
// sequence with past p and chunk length c sees keys 0 .. p + t (none when
// t >= c). Without MT, seq_lens holds the key counts and every head sees
// them all.
template <typename T, int D, bool MT, int HG>
__global__ __launch_bounds__(64 * decode_waves(D * sizeof(T))) void decode_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ rho, const T* __restrict__ kc,
    const T* __restrict__ vc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ past_lens, float* __restrict__ out, float* __restrict__ ws,
    unsigned* __restrict__ counters, int H_q, int H_kv, int G, int S_max, int ntok, int chunk,
    int num_splits, float scale_log2) {
  using P = Dec<T, D>;
  constexpr int HW = 4 * HG;                         // query heads per workgroup
  constexpr int NW = decode_waves(D * sizeof(T));    // waves per workgroup
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) float lds_state[NW][HW][4];  // m, l, bs, cref per head
  __shared__ __attribute__((aligned(16))) float lds_vec[NW][2][HW][D];  // A, C per head
  __shared__ __attribute__((aligned(16))) char k_lds[NW][P::KLDS];  // bf16: each wave's K block

  // Grid (KV head x head group, sequence, split): workgroups are dealt to
  // the 8 XCDs in linear order (x fastest), so every XCD gets the same
  // splits of a different set of streams (with 8 KV heads: one head of every
  // sequence), whatever the split count. With the split varying fastest, a
  // power-of-two split count put split s of every stream on one XCD, and the
  // mostly empty high splits of a ragged batch left some XCDs with far more
  // work than others.
  const int ngroups = (G + HW - 1) / HW;
  int hk = blockIdx.x / ngroups;
  int hgrp = blockIdx.x % ngroups;
  int b = blockIdx.y;
  int split = blockIdx.z;
  // Several head groups per KV head read the same K and V: place a KV head's
  // groups on one XCD, dispatched one after another, so the repeat reads are
  // served by that XCD's L2 (decode at 64 query heads on 8 KV heads: 43.4 ->
  // 32.1 us; 4 new tokens per sequence at G = 2: 44 -> 32.7 us).
  if (ngroups > 1) {
    const unsigned total = gridDim.x * gridDim.y * gridDim.z;
    if (total % (8u * (unsigned)ngroups) == 0u) {
      const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
      const unsigned k = lin / 8u;
      hgrp = (int)(k % (unsigned)ngroups);
      const unsigned rest = (k / (unsigned)ngroups) * 8u + lin % 8u;  // (KV head, b, split)
      hk = (int)(rest % (unsigned)H_kv);
      b = (int)((rest / (unsigned)H_kv) % gridDim.y);
      split = (int)(rest / ((unsigned)H_kv * gridDim.y));
    }
  }
  const int Gw = min(HW, G - HW * hgrp);             // heads in this workgroup
  const int h0 = hk * G + HW * hgrp;                 // first query head

  int n, past = 0, clen = 0;
  if constexpr (MT) {
    past = min(max(past_lens[b], 0), S_max);
    clen = min(max(seq_lens[b], 0), min(ntok, S_max - past));
    n = past + clen;
  } else {
    n = min(max(seq_lens[b], 0), S_max);
  }
  const int j0 = split * chunk;
  const bool direct = (num_splits == 1);
  const bool fused = counters != nullptr;            // last workgroup merges the splits
  if (j0 >= n && !direct) {                          // empty split: the merge skips it
    if (fused && n == 0 && split == 0) {             // no workgroup holds a key
      for (int idx = threadIdx.x; idx < Gw * D; idx += NT)
        out[((size_t)b * H_q + h0) * D + idx] = 0.f;
    }
    return;
  }
  const int j1 = min(j0 + chunk, n);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;                           // lane group (0..3)
  const int c = lane & 15;                           // lane column (0..15)
  const int hq = c >> 2;                             // head whose scores this lane holds
  const int t = c & 3;                               // 0,1: q / e rows; 2,3: rho / e*r rows
  // Heads 4 hg + hq (hg < HG) of the workgroup: with HG = 2 a second probe
  // tile (and a second set of value accumulators) serves four more heads
  // from the same K and V reads.
  // Keys each of this lane's heads sees: all n, or, per token, the causal prefix.
  int lim[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    lim[hg] = n;
    if constexpr (MT) {
      const int tok = (h0 + 4 * hg + hq) % ntok;
      lim[hg] = tok < clen ? past + tok + 1 : 0;
    }
  }

  // Probe operand (B of the score MFMA): column c, dims 32 kk + 8 g + (0..7).
  bf16x8 pr_hi[HG][P::KSTEPS], pr_lo[HG][P::KSTEPS];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const bool live = 4 * hg + hq < Gw;
    const T* src = (t < 2 ? q : rho) + ((size_t)b * H_q + h0 + (live ? 4 * hg + hq : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < P::KSTEPS; ++kk) {
      uint32_t w[P::KW];
      load_probe_words<T>(src + 32 * kk + 8 * g, P::KW, w);
      if (!live) {
#pragma unroll
        for (int i = 0; i < P::KW; ++i) w[i] = 0;
      }
      to_operand<T>(w, pr_hi[hg][kk], pr_lo[hg][kk]);
    }
  }

  const size_t slice = ((size_t)b * H_kv + hk) * (size_t)S_max * D;
  // The range ends at this workgroup's last key (j1 <= n): loads past it
  // return zeros without touching memory.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + slice, (uint32_t)j1 * P::ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + slice, (uint32_t)j1 * P::ROWB);

  f32x4 acc[HG][P::DPL];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) acc[hg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[HG], lsum[HG], cref[HG];  // per head 4 hg + hq: running max (log2 units),
#pragma unroll                       // this lane's part of l (t == 0) or Bs (t == 2),
  for (int hg = 0; hg < HG; ++hg) {  // and the probe reference
    m[hg] = -INFINITY;
    lsum[hg] = 0.f;
    cref[hg] = 0.f;
  }
  bool first = true;

  // K pieces for the score MFMA and V rows for the value MFMA of one block.
  // bf16: K is read in whole rows (piece i of lane l is 16-byte piece
  // l + 64 i of the block, row-major), with the streaming hint like V, and
  // rearranged through this wave's LDS region; fp32: each lane reads its
  // operand pieces (16 rows x 64 bytes per instruction) directly.
  auto load_block = [&](int blk, Words<P::KW> (&kw)[2][P::KSTEPS], Words<P::VW> (&vw)[8]) {
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2)
#pragma unroll
      for (int kk = 0; kk < P::KSTEPS; ++kk) {
        if constexpr (!P::F32) {
          const int pc = lane + 64 * (T2 * P::KSTEPS + kk);
          kw[T2][kk] = buffer_load<P::KW, kNontemporal>(
              krs, (uint32_t)(blk + pc / P::RP) * P::ROWB + (pc % P::RP) * 16);
        } else {
          kw[T2][kk] = buffer_load<P::KW>(
              krs, (uint32_t)(blk + 16 * T2 + c) * P::ROWB + (32 * kk + 8 * g) * P::ESZ);
        }
      }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vw[e] = buffer_load<P::VW, kNontemporal>(
          vrs, (uint32_t)(blk + 16 * (e >> 2) + 4 * g + (e & 3)) * P::ROWB + P::DPL * c * P::ESZ);
  };

  // Contracts block blk (its K and V pieces already in kw, vw).
  auto process = [&](int blk, const Words<P::KW> (&kw)[2][P::KSTEPS], const Words<P::VW> (&vw)[8]) {

    // bf16: the block's K rows into this wave's LDS region (rows padded by
    // 16 bytes), then the A operand of each score MFMA (key row 16 T2 + c,
    // dims 32 kk + 8 g .. + 7) read back. A wave's LDS accesses take effect in
    // order, so no barrier is needed.
    bf16x8 kop[2][P::KSTEPS];
    if constexpr (!P::F32) {
      char* kl = k_lds[wave];
#pragma unroll
      for (int T2 = 0; T2 < 2; ++T2)
#pragma unroll
        for (int kk = 0; kk < P::KSTEPS; ++kk) {
          const int pc = lane + 64 * (T2 * P::KSTEPS + kk);
          *reinterpret_cast<i32x4*>(kl + (pc / P::RP) * P::KSTR + (pc % P::RP) * 16) =
              __builtin_bit_cast(i32x4, kw[T2][kk]);
        }
#pragma unroll
      for (int T2 = 0; T2 < 2; ++T2)
#pragma unroll
        for (int kk = 0; kk < P::KSTEPS; ++kk)
          kop[T2][kk] = *reinterpret_cast<const bf16x8*>(kl + (16 * T2 + c) * P::KSTR + 64 * kk + 16 * g);
    }

    // ---- scores: lane (g, c) gets probe column c for keys 16 T2 + 4 g + i
    f32x4 sc[HG][2];
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2) {
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) sc[hg][T2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < P::KSTEPS; ++kk) {
        bf16x8 khi, klo;
        if constexpr (!P::F32)
          khi = kop[T2][kk];
        else
          to_operand<T>(kw[T2][kk].w, khi, klo);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          sc[hg][T2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khi, pr_hi[hg][kk], sc[hg][T2], 0, 0, 0);
          if constexpr (P::F32) {
            sc[hg][T2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khi, pr_lo[hg][kk], sc[hg][T2], 0, 0, 0);
            sc[hg][T2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(klo, pr_hi[hg][kk], sc[hg][T2], 0, 0, 0);
          }
        }
      }
    }

    const bool take_ref = first;
    first = false;
    bf16x8 aop[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      float x[8], rv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float raw = sc[hg][e >> 2][e & 3];
        const int key = blk + 16 * (e >> 2) + 4 * g + (e & 3);
        float s = quad_perm_0101(raw) * scale_log2;
        s = key < j1 && (!MT || key < lim[hg]) ? s : -INFINITY;
        x[e] = s;
        rv[e] = raw;
        mx = fmaxf(mx, s);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));

      if (take_ref) {
        // reference: r of the first key of this wave's first block (lane 4h+2, slot 0)
        cref[hg] = __shfl(rv[0], 4 * hq + 2);
      }

      const bool need = mx > m[hg] + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float mnew = need ? mx : m[hg];
        const float alpha = need ? exp2f(m[hg] - mnew) : 1.0f;
        m[hg] = mnew;
        lsum[hg] *= alpha;
        const float a_acc = __shfl(alpha, 4 * g);  // accumulator rows belong to head g
#pragma unroll
        for (int j = 0; j < P::DPL; ++j) acc[hg][j] *= a_acc;
      }

      // ---- value-MFMA A operand: row c = 4h + t, key slots (g, e)
      uint32_t aw[4];
      {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // With MT a head may have no visible key yet (m still -inf).
          const float p = (MT && x[e] == -INFINITY) ? 0.f : exp2f(x[e] - m[hg]);
          float val = t >= 2 ? p * (rv[e] - cref[hg]) : p;
          val = 4 * hg + hq < Gw ? val : 0.f;
          lsum[hg] += val;
          const float hi = bf16_round(val);
          a[e] = (t & 1) ? val - hi : val;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) aw[u] = pack_bf16(a[2 * u], a[2 * u + 1]);
      }
      aop[hg] = as_bf16x8(aw[0], aw[1], aw[2], aw[3]);
    }

    // ---- values: N-tile j covers dims (d/16) c + j
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      if constexpr (!P::F32) {
        uint32_t bw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          bw[u] = pair_halves(vw[2 * u].w[j >> 1], vw[2 * u + 1].w[j >> 1], j & 1);
        const bf16x8 bop = as_bf16x8(bw[0], bw[1], bw[2], bw[3]);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
          acc[hg][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[hg], bop, acc[hg][j], 0, 0, 0);
      } else {
        float vv[8], vr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vv[e] = __uint_as_float(vw[e].w[j]);
          vr[e] = vv[e] - bf16_round(vv[e]);
        }
        const bf16x8 bhi = as_bf16x8(pack_bf16(vv[0], vv[1]), pack_bf16(vv[2], vv[3]),
                                     pack_bf16(vv[4], vv[5]), pack_bf16(vv[6], vv[7]));
        const bf16x8 blo = as_bf16x8(pack_bf16(vr[0], vr[1]), pack_bf16(vr[2], vr[3]),
                                     pack_bf16(vr[4], vr[5]), pack_bf16(vr[6], vr[7]));
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          acc[hg][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[hg], bhi, acc[hg][j], 0, 0, 0);
          acc[hg][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[hg], blo, acc[hg][j], 0, 0, 0);
        }
      }
    }
  };

  for (int blk = j0 + kBlockKeys * wave; blk < j1; blk += kBlockKeys * NW) {
    Words<P::KW> kw[2][P::KSTEPS];
    Words<P::VW> vw[8];
    load_block(blk, kw, vw);
    process(blk, kw, vw);
  }

  // ---- per-wave state to LDS (a wave without blocks leaves l = 0)
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    float tot = lsum[hg] + __shfl_xor(lsum[hg], 16);
    tot += __shfl_xor(tot, 32);
    if (g == 0) {
      if (t == 0) {
        lds_state[wave][4 * hg + hq][0] = m[hg];
        lds_state[wave][4 * hg + hq][1] = first ? 0.f : tot;
        lds_state[wave][4 * hg + hq][3] = cref[hg];
      } else if (t == 2) {
        lds_state[wave][4 * hg + hq][2] = first ? 0.f : tot;
      }
    }
#pragma unroll
    for (int j = 0; j < P::DPL; ++j) {
      lds_vec[wave][0][4 * hg + g][P::DPL * c + j] = acc[hg][j][0] + acc[hg][j][1];
      lds_vec[wave][1][4 * hg + g][P::DPL * c + j] = acc[hg][j][2] + acc[hg][j][3];
    }
  }
  __syncthreads();

  // ---- merge the waves; finalise (one split) or write the partial record.
  // The records of this workgroup's heads lie in one range of the workspace
  // (heads h0 .. h0 + Gw - 1, every split), reached through one descriptor.
  // With the fused merge they are written and read at the device-coherent
  // level (kCoherent) instead of staying in this XCD's L2, so the merging
  // workgroup (on any XCD) reads them without any cache-wide write-back or
  // invalidate.
  float* const wbase = direct ? out : ws + ((size_t)b * H_q + h0) * num_splits * P::REC;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(wbase, direct ? 0u : (uint32_t)(Gw * num_splits * P::REC * 4));
  // V dimensions per thread, as many as keep the workgroup busy (1, 2 or
  // 4): wider LDS reads, record stores and record loads. Four only in the
  // 8-head instantiation (4 x 128 dims never reach 1024 items), so that the
  // 4-head kernel keeps its register count (164: three workgroups per
  // compute unit in long, ragged batches).
  const int V = (HG == 2 && Gw * D >= 1024) ? 4 : (Gw * D >= 512 ? 2 : 1);
  // Waves merge in LDS. Branch-free: every LDS read of an item is issued
  // before any is used (the state of each wave as one 16-byte read),
  // waves without keys (l = 0) get weight 0, and the reference c0 is the
  // first wave's with keys.
  auto wave_merge = [&](auto vtag) {
    constexpr int VV = decltype(vtag)::value;
    using VT = typename Vec<VV>::T;
    for (int idx = tid; idx < Gw * D / VV; idx += NT) {
      const int h = idx / (D / VV);
      const int q = idx % (D / VV);
      float4 st[NW];  // m, l, bs, cref
      VT Aw[NW], Cw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        st[w] = *reinterpret_cast<const float4*>(&lds_state[w][h][0]);
        Aw[w] = *reinterpret_cast<const VT*>(&lds_vec[w][0][h][VV * q]);
        Cw[w] = *reinterpret_cast<const VT*>(&lds_vec[w][1][h][VV * q]);
      }
      float M = -INFINITY;
      float c0 = 0.f;
#pragma unroll
      for (int w = NW - 1; w >= 0; --w) {
        M = st[w].y > 0.f ? fmaxf(M, st[w].x) : M;
        c0 = st[w].y > 0.f ? st[w].w : c0;
      }
      float l = 0.f, bs = 0.f;
      VT A{}, C{};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float lw = st[w].y;
        const float al = lw > 0.f ? exp2f(st[w].x - M) : 0.f;
        const float sh = st[w].w - c0;
        l += al * lw;
        bs += al * (st[w].z + sh * lw);
        A += al * Aw[w];
        C += al * (Cw[w] + sh * Aw[w]);
      }
      if (direct) {
        *reinterpret_cast<VT*>(out + ((size_t)b * H_q + h0 + h) * D + VV * q) =
            l > 0.f ? (A * (1.f + bs / l) - C) / l : VT{};
      } else {
        const uint32_t rec = (uint32_t)((h * num_splits + split) * P::REC * 4);
        const f32x4 hd = {M, l, bs, c0};
        if (fused) {
          if (q == 0) hdr_store<true>(hd, wbase, wrs, rec);
          rec_store<VV, true>(A, wbase, wrs, rec + 16 + 4 * VV * q);
          rec_store<VV, true>(C, wbase, wrs, rec + 16 + 4 * D + 4 * VV * q);
        } else {
          if (q == 0) hdr_store<false>(hd, wbase, wrs, rec);
          rec_store<VV, false>(A, wbase, wrs, rec + 16 + 4 * VV * q);
          rec_store<VV, false>(C, wbase, wrs, rec + 16 + 4 * D + 4 * VV * q);
        }
      }
    }
  };
  if (HG == 2 && V == 4)
    wave_merge(std::integral_constant<int, 4 * HG / 2>{});
  else if (V == 2)
    wave_merge(std::integral_constant<int, 2>{});
  else
    wave_merge(std::integral_constant<int, 1>{});
  if (direct || !fused) return;

  // ---- fused merge: the workgroup that finishes last for this (b, KV head,
  // head group) merges every split's record. Each thread waits until its own
  // coherent record stores have completed before the workgroup barrier, so
  // they are performed before thread 0's arrival increment; the last arrival
  // reads the records at the coherent level and returns the counter to zero.
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    unsigned* ctr = counters + ((size_t)b * H_kv + hk) * ngroups + hgrp;
    const unsigned nsv = (unsigned)((n + chunk - 1) / chunk);
    const unsigned prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev + 1 == nsv);
    if (s_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  const int nsv = (n + chunk - 1) / chunk;
  auto split_merge = [&](auto vtag) {
    constexpr int VV = decltype(vtag)::value;
    using VT = typename Vec<VV>::T;
    for (int idx = tid; idx < Gw * D / VV; idx += NT) {  // (head, VV dims)
      const int h = idx / (D / VV);
      const int q = idx % (D / VV);
      *reinterpret_cast<VT*>(out + ((size_t)b * H_q + h0 + h) * D + VV * q) =
          merge_splits<D, VV, true>(wbase, wrs, (uint32_t)(h * num_splits * P::REC * 4), nsv, q);
    }
  };
  if (HG == 2 && V == 4)
    split_merge(std::integral_constant<int, 4 * HG / 2>{});
  else  // pairs at least (the single-float form measured slower)
    split_merge(std::integral_constant<int, 2>{});
}

// One workgroup of D/4 threads per (b, h_q): merges the partial records of
// the splits that hold keys and writes out[b, h_q, :].
template <int D>
__global__ __launch_bounds__(32) void decode_combine_kernel(const int32_t* __restrict__ seq_lens,
                                                             const float* __restrict__ ws,
                                                             float* __restrict__ out, int H_q,
                                                             int S_max, int chunk, int num_splits) {
  constexpr int REC = 2 * D + 4;
  const int bh = blockIdx.x;
  const int b = bh / H_q;
  const int n = min(max(seq_lens[b], 0), S_max);
  const int nsv = min(num_splits, (n + chunk - 1) / chunk);
  const float* base = ws + (size_t)bh * num_splits * REC;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint32_t)(num_splits * REC * 4));
  *reinterpret_cast<f32x4*>(out + (size_t)bh * D + 4 * threadIdx.x) =
      merge_splits<D, 4, false>(base, r, 0u, nsv, threadIdx.x);
}

template <typename T, int D, bool MT, int HG>
hipError_t launch_partial_hg(const DecodeArgs& a, hipStream_t st) {
  const int ngroups = (a.G + 4 * HG - 1) / (4 * HG);
  dim3 grid(a.H_kv * ngroups, a.B, a.num_splits);  // stream fastest in the linear order
  hipLaunchKernelGGL((decode_partial_kernel<T, D, MT, HG>), grid, dim3(64 * decode_waves(D * sizeof(T))), 0, st,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.rho),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.seq_lens,
                     a.past_lens, a.out, static_cast<float*>(a.ws),
                     static_cast<unsigned*>(a.counters), a.H_q, a.H_kv, a.G, a.S_max, a.ntok,
                     a.chunk, a.num_splits, a.scale * kLog2e);
  return hipGetLastError();
}

template <typename T, int D, bool MT>
hipError_t launch_partial_t(const DecodeArgs& a, hipStream_t st) {
  return decode_heads_per_workgroup(a.G) == 8 ? launch_partial_hg<T, D, MT, 2>(a, st)
                                              : launch_partial_hg<T, D, MT, 1>(a, st);
}

template <bool MT>
hipError_t launch_partial_mt(const DecodeArgs& a, hipStream_t st) {
  if (a.f32)
    return a.d == 64 ? launch_partial_t<float, 64, MT>(a, st) : launch_partial_t<float, 128, MT>(a, st);
  return a.d == 64 ? launch_partial_t<__bf16, 64, MT>(a, st) : launch_partial_t<__bf16, 128, MT>(a, st);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t st) {
  return a.past_lens ? launch_partial_mt<true>(a, st) : launch_partial_mt<false>(a, st);
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H_q);
  if (a.d == 64) {
    hipLaunchKernelGGL((decode_combine_kernel<64>), grid, dim3(16), 0, st, a.seq_lens,
                       static_cast<const float*>(a.ws), a.out, a.H_q, a.S_max, a.chunk,
                       a.num_splits);
  } else {
    hipLaunchKernelGGL((decode_combine_kernel<128>), grid, dim3(32), 0, st, a.seq_lens,
                       static_cast<const float*>(a.ws), a.out, a.H_q, a.S_max, a.chunk,
                       a.num_splits);
  }
  return hipGetLastError();
}

}  // namespace parallax
