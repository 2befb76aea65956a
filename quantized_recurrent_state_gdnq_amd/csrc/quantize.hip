// Row codec on gfx950: per row (d_k fp32 entries, optionally rotated by the
// normalised Walsh-Hadamard matrix first), scale = absmax / 127 and codes =
// clamp(round_half_even(x / scale), -127, 127); an all-zero row gets scale 0.
// The 4-bit state takes absmax / 7 and [-7, 7], two codes per byte.
// LeapQuant (abstract): the 8-bit recurrent state; LinQuant / Influence-
// Inspired Spectral Rotations (abstracts): the WHT rotation.
//
// 16 lanes per row, E = d_k / 16 consecutive entries per lane (16-byte
// loads), 16 rows per 256-thread workgroup; absmax by DPP inside the row.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace gdnq {

constexpr int Q_THREADS = 256;
constexpr int Q_LPR = 16;

template <int DK, bool WHT, int QB>
__global__ __launch_bounds__(Q_THREADS) void quantize_kernel(const float* __restrict__ S,
                                                             int64_t rows,
                                                             int8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  constexpr int E = DK / Q_LPR;  // 8 or 4
  const int tid = threadIdx.x;
  const int li = tid % Q_LPR;
  const int64_t row = int64_t(blockIdx.x) * (Q_THREADS / Q_LPR) + tid / Q_LPR;
  const bool valid = row < rows;
  float v[E];
  if (valid) {
    const float4* src = reinterpret_cast<const float4*>(S + row * DK + li * E);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 x = src[i];
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = 0.f;
  }
  if constexpr (WHT) fwht_group<E, Q_LPR>(v, li);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<Q_LPR>(amax);
  constexpr int QMAX = QB == 8 ? 127 : 7;
  const float scale = codec_scale<QMAX>(amax);
  if (!valid) return;
  float cf[E];  // the reciprocal form: the codes of one division per element
  codec_codes<E, QMAX>(v, scale, cf);
  if constexpr (QB == 8) {
    uint32_t w[E / 4];
#pragma unroll
    for (int i = 0; i < E / 4; ++i)
      w[i] = pack4_i8(int(cf[4 * i]), int(cf[4 * i + 1]), int(cf[4 * i + 2]), int(cf[4 * i + 3]));
    int8_t* dst = codes + row * DK + li * E;
    if constexpr (E == 8) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    }
  } else {  // E codes in E / 2 bytes
    int c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < E; ++i) c[i] = int(cf[i]);
    const uint32_t w = pack8_i4(c);
    int8_t* dst = codes + row * (DK / 2) + li * (E / 2);
    if constexpr (E == 8) {
      *reinterpret_cast<uint32_t*>(dst) = w;
    } else {
      *reinterpret_cast<uint16_t*>(dst) = uint16_t(w);
    }
  }
  if (li == 0) scales[row] = scale;
}

template <int DK, int QB>
static void launch_q(const QuantizeLaunch& L, unsigned grid, hipStream_t stream) {
  if (L.wht)
    hipLaunchKernelGGL((quantize_kernel<DK, true, QB>), dim3(grid), dim3(Q_THREADS), 0, stream, L.S, L.rows,
                       L.codes, L.scales);
  else
    hipLaunchKernelGGL((quantize_kernel<DK, false, QB>), dim3(grid), dim3(Q_THREADS), 0, stream, L.S, L.rows,
                       L.codes, L.scales);
}

hipError_t launch_quantize(const QuantizeLaunch& L, hipStream_t stream) {
  const int64_t rows_per_blk = Q_THREADS / Q_LPR;
  const unsigned grid = unsigned((L.rows + rows_per_blk - 1) / rows_per_blk);
  if (L.d_k == 128)
    L.q4 ? launch_q<128, 4>(L, grid, stream) : launch_q<128, 8>(L, grid, stream);
  else
    L.q4 ? launch_q<64, 4>(L, grid, stream) : launch_q<64, 8>(L, grid, stream);
  return hipGetLastError();
}
}  // namespace gdnq
