// bf16 MFMA helpers for gfx950 (v_mfma_f32_16x16x32_bf16).
//
// Lane layout of one 16x16x32 product D[16][16] += A[16][32] * B[32][16]:
//   A: lane l holds row (l % 16), k = 8 * (l / 16) .. +8   (8 bf16)
//   B: lane l holds column (l % 16), k = 8 * (l / 16) .. +8 (8 bf16)
//   D: lane l holds column (l % 16), rows 4 * (l / 16) .. +4 (4 fp32)
// Storing every operand k-contiguous ([row][k] for A, [column][k] for B)
// makes each fragment one 16-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdnq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 8 int8 codes -> 8 bf16 (exact: |code| <= 127)
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint2 w) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)float(int32_t(w.x << (24 - 8 * e)) >> 24);
    r[4 + e] = (__bf16)float(int32_t(w.y << (24 - 8 * e)) >> 24);
  }
  return r;
}

// x = hi + mid + lo with each part a bf16: hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid).  The three carry 24 significant bits, so a product
// with an exact bf16 operand summed over the three parts matches fp32.
template <int N, typename V>
__device__ __forceinline__ void split3(const float (&x)[N], V& hi, V& mid, V& lo) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const __bf16 h = (__bf16)x[e];
    const float r1 = x[e] - float(h);
    const __bf16 m = (__bf16)r1;
    hi[e] = h;
    mid[e] = m;
    lo[e] = (__bf16)(r1 - float(m));
  }
}

// x = hi + lo (16 significant bits)
template <int N, typename V>
__device__ __forceinline__ void split2(const float (&x)[N], V& hi, V& lo) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - float(h));
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// The same splits taken by truncation, for even N: hi keeps the upper 16 bits
// of x, mid those of r = x - hi (exact), lo is r - mid (exact, at most eight
// significant bits left).  hi + mid + lo equals x exactly; hi + mid keeps 16
// significant bits.  One AND and one subtraction per part and element, and a
// byte permute per pair packs the upper halves.
template <int N, typename V>
__device__ __forceinline__ void split3t(const float (&x)[N], V& hi, V& mid, V& lo) {
  typedef uint32_t W __attribute__((ext_vector_type(N / 2)));
  W h2, m2, l2;
#pragma unroll
  for (int e = 0; e < N; e += 2) {
    const uint32_t a0 = __float_as_uint(x[e]), a1 = __float_as_uint(x[e + 1]);
    const float r0 = x[e] - __uint_as_float(a0 & 0xffff0000u), r1 = x[e + 1] - __uint_as_float(a1 & 0xffff0000u);
    const uint32_t b0 = __float_as_uint(r0), b1 = __float_as_uint(r1);
    const float s0 = r0 - __uint_as_float(b0 & 0xffff0000u), s1 = r1 - __uint_as_float(b1 & 0xffff0000u);
    h2[e / 2] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    m2[e / 2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
    l2[e / 2] = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
  }
  hi = __builtin_bit_cast(V, h2);
  mid = __builtin_bit_cast(V, m2);
  lo = __builtin_bit_cast(V, l2);
}

template <int N, typename V>
__device__ __forceinline__ void split2t(const float (&x)[N], V& hi, V& lo) {
  typedef uint32_t W __attribute__((ext_vector_type(N / 2)));
  W h2, l2;
#pragma unroll
  for (int e = 0; e < N; e += 2) {
    const uint32_t a0 = __float_as_uint(x[e]), a1 = __float_as_uint(x[e + 1]);
    const float r0 = x[e] - __uint_as_float(a0 & 0xffff0000u), r1 = x[e + 1] - __uint_as_float(a1 & 0xffff0000u);
    h2[e / 2] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    l2[e / 2] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
  }
  hi = __builtin_bit_cast(V, h2);
  lo = __builtin_bit_cast(V, l2);
}

}  // namespace gdnq
