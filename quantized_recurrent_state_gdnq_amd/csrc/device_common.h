// Device helpers shared by the gfx950 kernels: bf16 conversion, wave-level
// reductions (DPP inside a row of 16 lanes, cross-row swizzles above), the
// register/cross-lane fast Walsh-Hadamard transform and the int8 row codec.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdnq {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}
// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- DPP / reductions
// DPP control words (GFX9 encoding).
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// DPP move with a row mask: rows left out, and lanes whose source falls
// outside the row, read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP: row_shr by
// 1, 2, 4, 8 inside each row of 16, then row_bcast:15 adds the last lane of
// rows 0 and 2 to rows 1 and 3, and row_bcast:31 adds lane 31 to rows 2, 3.
__device__ __forceinline__ float wave_scan_incl(float x) {
  x += dpp_rows<0x111, 0xF>(x);
  x += dpp_rows<0x112, 0xF>(x);
  x += dpp_rows<0x114, 0xF>(x);
  x += dpp_rows<0x118, 0xF>(x);
  x += dpp_rows<0x142, 0xA>(x);
  x += dpp_rows<0x143, 0xC>(x);
  return x;
}

// Lanes l and l ^ 16 (v_permlane16_swap: rows 0 <-> 1, 2 <-> 3) and lanes l
// and l ^ 32 (v_permlane32_swap: halves), on the VALU (gfx950): each returns
// the pair (value of the lower lane, value of the upper lane), so a
// commutative combination of the two is the same in both lanes.
__device__ __forceinline__ float xor16_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Sum over aligned groups of N consecutive lanes (N = 1..64); every lane of a
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<DPP_XOR1>(x);
  if constexpr (N >= 4) x += dpp<DPP_XOR2>(x);
  if constexpr (N >= 8) x += dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x = xor16_sum(x);
  if constexpr (N >= 64) x = xor32_sum(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<DPP_XOR1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<DPP_XOR2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<DPP_ROW_MIRROR>(x));
  if constexpr (N >= 32) x = xor16_max(x);
  if constexpr (N >= 64) x = xor32_max(x);
  return x;
}

// Full-wave sum returned as a wave-uniform value: DPP inside each row of 16
// lanes, then the four row sums are read out of lanes 0/16/32/48.
__device__ __forceinline__ float wave_sum_uniform(float x) {
  x = group_sum<16>(x);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (a + b) + (c + d);
}

// Full-wave sum in every lane, all in VALU: DPP inside each row of 16 lanes,
// then v_permlane16_swap (row pairs) and v_permlane32_swap (halves), gfx950.
__device__ __forceinline__ float wave_allreduce_sum(float x) {
  x = group_sum<16>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Three independent full-wave sums, stage by stage, so that their latencies
// overlap.
// Three independent full-wave sums returned as wave-uniform values: DPP
// inside each row of 16, then row_bcast:15 / row_bcast:31 fold the row sums
// into lane 63, which is read into a scalar register.  The additions pair the
// row sums as (r0 + r1) + (r2 + r3), as wave_allreduce_sum3 does.
__device__ __forceinline__ void wave_sum3_uniform(float& x, float& y, float& z) {
  x += dpp<DPP_XOR1>(x);
  y += dpp<DPP_XOR1>(y);
  z += dpp<DPP_XOR1>(z);
  x += dpp<DPP_XOR2>(x);
  y += dpp<DPP_XOR2>(y);
  z += dpp<DPP_XOR2>(z);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  y += dpp<DPP_ROW_HALF_MIRROR>(y);
  z += dpp<DPP_ROW_HALF_MIRROR>(z);
  x += dpp<DPP_ROW_MIRROR>(x);
  y += dpp<DPP_ROW_MIRROR>(y);
  z += dpp<DPP_ROW_MIRROR>(z);
  // rows 1, 3 += lane 15 of rows 0, 2; then rows 2, 3 += lane 31.  Rows left
  // out of the row mask keep their value, so each stage is one DPP add (the
  // compiler emits a move and an add for the masked form).  The leading
  // s_nop covers the two wait states a DPP read of a just-written VGPR needs;
  // the second stage of each value is three instructions after its first.
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %2, %2 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %2, %2 row_bcast:31 row_mask:0xc bank_mask:0xf"
      : "+v"(x), "+v"(y), "+v"(z));
  x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(y), 63));
  z = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 63));
}

__device__ __forceinline__ void wave_allreduce_sum3(float& x, float& y, float& z) {
  x += dpp<DPP_XOR1>(x);
  y += dpp<DPP_XOR1>(y);
  z += dpp<DPP_XOR1>(z);
  x += dpp<DPP_XOR2>(x);
  y += dpp<DPP_XOR2>(y);
  z += dpp<DPP_XOR2>(z);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  y += dpp<DPP_ROW_HALF_MIRROR>(y);
  z += dpp<DPP_ROW_HALF_MIRROR>(z);
  x += dpp<DPP_ROW_MIRROR>(x);
  y += dpp<DPP_ROW_MIRROR>(y);
  z += dpp<DPP_ROW_MIRROR>(z);
  const auto a1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const auto b1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  const auto c1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  x = __uint_as_float(a1[0]) + __uint_as_float(a1[1]);
  y = __uint_as_float(b1[0]) + __uint_as_float(b1[1]);
  z = __uint_as_float(c1[0]) + __uint_as_float(c1[1]);
  const auto a2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  const auto c2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  x = __uint_as_float(a2[0]) + __uint_as_float(a2[1]);
  y = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
  z = __uint_as_float(c2[0]) + __uint_as_float(c2[1]);
}

// ---------------------------------------------------------------- FWHT
// Fast Walsh-Hadamard transform of a d-vector spread over a group of lanes:
// lane j of the group holds elements [j*E, j*E + E) in v[0..E).  The
// butterfly (x_i, x_{i+s}) -> (x_i + x_{i+s}, x_i - x_{i+s}) over every
// stride s = 1, 2, ..., d/2 yields H x with H the Sylvester Hadamard matrix
// H[i][j] = (-1)^popcount(i & j); the result is then scaled by 1/sqrt(d).
// The group is `lanes = d / E` consecutive lanes, aligned.
template <int E>
__device__ __forceinline__ void fwht_local(float (&v)[E]) {
#pragma unroll
  for (int s = 1; s < E; s <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if ((i & s) == 0) {
        float a = v[i], b = v[i + s];
        v[i] = a + b;
        v[i + s] = a - b;
      }
    }
  }
}

template <int E, int LANES>
__device__ __forceinline__ void fwht_group(float (&v)[E], int lane_in_group) {
  fwht_local<E>(v);
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) {
    const bool upper = (lane_in_group & m) != 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float other = __shfl_xor(v[i], m, 64);
      v[i] = upper ? (other - v[i]) : (v[i] + other);
    }
  }
  constexpr float inv_sqrt = (E * LANES == 128) ? 0.08838834764831845f
                             : (E * LANES == 64) ? 0.125f
                             : (E * LANES == 256) ? 0.0625f
                                                  : 0.0f;
  static_assert(inv_sqrt != 0.0f, "unsupported FWHT length");
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] *= inv_sqrt;
}

// ---------------------------------------------------------------- codec
// scale = absmax / 127 (IEEE division); code = clamp(rne(x / scale), -127, 127).
// QMAX = 127: the 8-bit state; QMAX = 7: the uniform 4-bit state (15
// levels, two codes per byte).  Same rule, scale = absmax / QMAX.
template <int QMAX = 127>
__device__ __forceinline__ float codec_scale(float absmax) { return __fdiv_rn(absmax, float(QMAX)); }

template <int QMAX = 127>
__device__ __forceinline__ int codec_code(float x, float scale) {
  if (scale == 0.0f) return 0;
  float r = __builtin_rintf(__fdiv_rn(x, scale));
  r = fminf(fmaxf(r, -float(QMAX)), float(QMAX));
  return int(r);
}

// Codes of N elements of one row, as floats, equal element by element to
// codec_code.  With inv = fl(1/scale), q = fl(x * inv) is within
// |x/scale| * 2^-23 <= 1.6e-5 of the exact quotient and fl(x/scale) within
// 7.6e-6 of it, so their nearest integers can differ only when q lies within
// 2.4e-5 of a half-integer; only then (rarely) the IEEE divisions are done.
// A subnormal scale below 2^-128 has no finite reciprocal (and subnormal
// scales carry fewer significant bits): such rows always divide.
template <int N, int QMAX = 127>
__device__ __forceinline__ void codec_codes(const float (&x)[N], float scale, float (&c)[N]) {
  const float inv = scale > 0.0f ? __frcp_rn(scale) : 0.0f;
  bool near = scale > 0.0f && scale < 1.17549435e-38f;  // subnormal: divide
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float q = x[e] * inv;
    const float r = __builtin_rintf(q);
    near |= fabsf(fabsf(q - r) - 0.5f) < 3.0e-5f;
    c[e] = r;
  }
  if (near) {
#pragma unroll
    for (int e = 0; e < N; ++e) c[e] = __builtin_rintf(__fdiv_rn(x[e], scale));
  }
#pragma unroll
  for (int e = 0; e < N; ++e) c[e] = fminf(fmaxf(c[e], -float(QMAX)), float(QMAX));
}

// The same codes from the row's absmax: scale = fl(absmax / QMAX) and
// inv = fl(QMAX / absmax), two independent divisions.  inv is within 2^-23
// (relative) of 1 / scale, so q = fl(x * inv) is within |x/scale| 1.8e-7 <=
// 2.3e-5 of the exact quotient and fl(x/scale) within 7.6e-6: their nearest
// integers can differ only when q lies within 3.1e-5 of a half-integer, and
// those rows divide.  A row whose scale rounds to 0 (absmax / QMAX below half
// the smallest subnormal) gets codes 0, as codec_code gives it.  Returns the
// scale.
template <int N, int QMAX = 127>
__device__ __forceinline__ float codec_row(const float (&x)[N], float absmax, float (&c)[N]) {
  const float scale = codec_scale<QMAX>(absmax);
  const float inv = scale > 0.0f ? __fdiv_rn(float(QMAX), absmax) : 0.0f;
  bool near = scale > 0.0f && scale < 1.17549435e-38f;  // subnormal: divide
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float q = x[e] * inv;
    const float r = __builtin_rintf(q);
    near |= fabsf(fabsf(q - r) - 0.5f) < 4.0e-5f;
    c[e] = r;
  }
  if (near) {
#pragma unroll
    for (int e = 0; e < N; ++e) c[e] = __builtin_rintf(__fdiv_rn(x[e], scale));
  }
#pragma unroll
  for (int e = 0; e < N; ++e) c[e] = fminf(fmaxf(c[e], -float(QMAX)), float(QMAX));
  return scale;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t(a) & 0xffu) | ((uint32_t(b) & 0xffu) << 8) | ((uint32_t(c) & 0xffu) << 16) |
         ((uint32_t(d) & 0xffu) << 24);
}

__device__ __forceinline__ float i8_at(uint32_t w, int byte) {
  return float(int32_t(w << (24 - 8 * byte)) >> 24);
}

// 4-bit codes: eight per 32-bit word, code n in bits [4n, 4n + 4) as a two's
// complement nibble (column 2j in the low nibble of byte j)
__device__ __forceinline__ uint32_t pack8_i4(const int (&c)[8]) {
  uint32_t w = 0u;
#pragma unroll
  for (int n = 0; n < 8; ++n) w |= (uint32_t(c[n]) & 0xfu) << (4 * n);
  return w;
}

__device__ __forceinline__ float i4_at(uint32_t w, int n) {
  return float(int32_t(w << (28 - 4 * n)) >> 28);
}

// code n of a word holding 32 / QB codes of QB bits
template <int QB>
__device__ __forceinline__ float code_at(uint32_t w, int n) {
  if constexpr (QB == 8) return i8_at(w, n);
  else return i4_at(w, n);
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads through a resource whose size limits the access: a lane
// whose byte offset is at or past `nbytes` reads 0 and causes no memory
// traffic.  This predicates loads without branches (dword 3 = 0x00020000 is
// the gfx9-family raw-buffer format word).
// POL is the load's cache policy: 0, or BUF_STREAM (nontemporal) for data
// read once and not again soon.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int BUF_STREAM = 2;  // the nontemporal cache-policy bit of a buffer load
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
template <int POL = 0>
__device__ __forceinline__ float4 bload_f4(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, POL);
  float4 f;
  __builtin_memcpy(&f, &v, 16);
  return f;
}
template <int POL = 0>
__device__ __forceinline__ uint4 bload_u4(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, POL);
  uint4 u;
  __builtin_memcpy(&u, &v, 16);
  return u;
}
template <int POL = 0>
__device__ __forceinline__ uint2 bload_u2(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL);
  uint2 u;
  __builtin_memcpy(&u, &v, 8);
  return u;
}
template <int POL = 0>
__device__ __forceinline__ float bload_f1(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL));
}
// per-lane offset plus a scalar offset (wave-uniform)
template <int POL = 0>
__device__ __forceinline__ uint2 bload_u2s(rsrc_t r, uint32_t off, uint32_t soff) {
  auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, POL);
  uint2 u;
  __builtin_memcpy(&u, &v, 8);
  return u;
}
template <int POL = 0>
__device__ __forceinline__ float bload_f1s(rsrc_t r, uint32_t off, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, POL));
}
template <int POL = 0>
__device__ __forceinline__ uint32_t bload_h1s(rsrc_t r, uint32_t off, uint32_t soff) {  // 16 bits, zero-extended
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, POL);
}
template <int POL = 0>
__device__ __forceinline__ uint32_t bload_b1s(rsrc_t r, uint32_t off, uint32_t soff) {  // 8 bits, zero-extended
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, soff, POL);
}

// Nearest OCP FP8 E4M3 value of q (1 sign bit, 4 exponent bits with bias 7,
// 3 mantissa bits, largest finite 448), ties to even.  For |q| in
// [2^e, 2^(e+1)), e >= -6, the grid step is 2^(e-3); below 2^-6 it is 2^-9.
// Scaling by a power of two is exact, so rint (ties to even) on |q| / step
// rounds exactly; the result is a grid value, which the hardware conversion
// then encodes without rounding.  |q| <= 448 here (it saturates above).
__device__ __forceinline__ float e4m3_round(float q) {
  const float a = fabsf(q);
  const int be = int((__float_as_uint(a) >> 23) & 0xFFu);  // 0 for zero and fp32 subnormals
  const int e = be - 127 > -6 ? be - 127 : -6;
  const float r = fminf(ldexpf(rintf(ldexpf(a, 3 - e)), e - 3), 448.f);
  return copysignf(r, q);
}
// two E4M3 grid values -> their two bytes (low 16 bits); exact on grid values
__device__ __forceinline__ uint32_t e4m3_pack2(float lo, float hi) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false)) & 0xFFFFu;
}
// bytes 0, 1 (sel false) or 2, 3 (sel true) of w -> two floats (exact)
__device__ __forceinline__ float2 e4m3_unpack2(uint32_t w, bool sel) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = sel ? __builtin_amdgcn_cvt_pk_f32_fp8(int(w), true) : __builtin_amdgcn_cvt_pk_f32_fp8(int(w), false);
  return make_float2(v[0], v[1]);
}

// XCD-aware workgroup id: workgroups are dispatched round-robin over the 8
// XCDs, so block x runs on XCD x % 8.  This remaps ids so that consecutive
// logical ids share one XCD (and its L2): logical = (x % 8) * (n / 8) + x / 8.
// Valid when n is a multiple of 8; otherwise the identity is used.
__device__ __forceinline__ int xcd_swizzle(int x, int n) {
  if (n & 7) return x;
  return (x & 7) * (n >> 3) + (x >> 3);
}

}  // namespace gdnq
