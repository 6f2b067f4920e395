// Device helpers shared by the Parallax HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace parallax {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Buffer resource over [base, base + bytes): loads at offsets past `bytes`
// return zeros instead of touching memory (CDNA raw-buffer range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Loads of 4 * N bytes at byte offset `off` through a buffer resource.
template <int N>
struct Words {
  uint32_t w[N];
};

// Cache-policy operand of a buffer load: 0 = default, kNontemporal = the
// streaming hint for data read once (CDNA3/4 "nt" bit).
constexpr int kNontemporal = 2;

template <int N, int AUX = 0>
__device__ __forceinline__ Words<N> buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Words<N> out;
  if constexpr (N == 8) {
    i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    i32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, AUX);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out.w[i] = (uint32_t)a[i];
      out.w[4 + i] = (uint32_t)b[i];
    }
  } else if constexpr (N == 4) {
    i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
#pragma unroll
    for (int i = 0; i < 4; ++i) out.w[i] = (uint32_t)a[i];
  } else if constexpr (N == 2) {
    i32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    out.w[0] = (uint32_t)a[0];
    out.w[1] = (uint32_t)a[1];
  } else {
    static_assert(N == 1, "unsupported load width");
    out.w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  }
  return out;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 value rounded to bf16 and back (the "hi" part of a hi+lo split).
__device__ __forceinline__ float bf16_round(float a) {
  return __uint_as_float(pack_bf16(a, 0.0f) << 16);
}

// Packs the low (sel == 0) or high (sel == 1) bf16 halves of x and y as
// {x_half, y_half} (x in the low 16 bits).
__device__ __forceinline__ uint32_t pair_halves(uint32_t x, uint32_t y, int sel) {
  return sel ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  i32x4 v = {(int)a, (int)b, (int)c, (int)d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float quad_perm_0101(float v) {
  // lane t of each quad takes lane (t & 1)'s value
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x44, 0xf, 0xf, false));
}

}  // namespace parallax
