// Decode step of the per-window int8-state gated delta rule on gfx950.
//
// LeapQuant (abstract): inside a window the output comes from the fixed
// low-bit state plus the window's buffered high-precision writes, and the
// state is requantized once, when the window closes.  Low-Bit GDN ...
// (abstract): the buffered writes go through the full GDN transition.
//
// Open window (f + 1 < W), one 256-thread workgroup per (sequence, head):
//   with A_j = alpha_j (I - beta_j k_j k_j^T) (symmetric), the replay
//   S_t = S_0 A_1..A_t + sum_j beta_j v_j k_j^T A_{j+1}..A_t gives
//       o = S_t q = S_0 y_0 + sum_j c_j v_j,
//       y = q, then for j = t, t-1, ..., 1:  c_j = beta_j (k_j . y),
//                                             y <- alpha_j (y - c_j k_j),
//   so the d_v x d_k state is read once, as int8, and never rebuilt.
//   Wave 0 runs that backward sweep over the buffered keys (staged in LDS);
//   the other waves have already issued the int8 rows and buffered values.
// Window close (f + 1 == W), R workgroups per head, each owning d_v / R rows
//   (rows of the state evolve independently): replay the W writes on the
//   dequantized rows in fp32, take the output from that state, requantize
//   the rows (absmax/127, round-half-even) in place.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace gdnq {

constexpr int DEC_THREADS = 256;
constexpr int DEC_R = 8;  // workgroups per head (row split) for the window close

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  int8_t* codes;
  float* scales;
  float* buf_k;
  float* buf_v;
  float* buf_alpha;
  float* buf_beta;
  const int32_t* fill_in;
  int32_t* fill_out;
  void* o;
  int B, H, W;
};

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if constexpr (BF16) return bf16_at(static_cast<const uint16_t*>(p), i);
  else return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* p, size_t i, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(p)[i] = uint16_t(f32_to_bf16_bits(x));
  else static_cast<float*>(p)[i] = x;
}

// LDS layout (floats), shared by both paths; the host sizes it with the same
// formula (decode_lds_bytes).
template <int DK, int DV>
struct DecLds {
  static constexpr int RW = DV / DEC_R;
  __device__ static int k_off() { return 0; }                  // [W][DK] keys
  __device__ static int ab_off(int W) { return W * DK; }       // alpha[64], beta[64]
  __device__ static int y_off(int W) { return W * DK + 128; }  // [DK] y (open) / q (close)
  __device__ static int c_off(int W) { return W * DK + 128 + DK; }       // [64] c_j
  __device__ static int v_off(int W) { return W * DK + 192 + DK; }  // partial sums [NT*4] | v rows [W][RW]
  __device__ static int dot_off(int W) {
    const int vsz = (4 * DEC_THREADS > W * RW) ? 4 * DEC_THREADS : W * RW;
    return W * DK + 192 + DK + vsz;
  }
};

template <int DK, int DV, bool IN_BF16, bool OUT_BF16, bool WHT>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(DecodeArgs a) {
  constexpr int NT = DEC_THREADS;
  constexpr int EK = DK / 64;  // elements of a d_k vector per lane in a wave
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);

  const int nblk = a.B * a.H * DEC_R;
  const int logical = xcd_swizzle(blockIdx.x, nblk);
  const int bh = logical / DEC_R;
  const int r = logical % DEC_R;
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int W = a.W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int f = a.fill_in[b];
  f = f < 0 ? 0 : (f > W - 1 ? W - 1 : f);  // out-of-range fill is a data error; stay in bounds
  const bool closing = (f + 1 == W);
  if (!closing && r != 0) return;

  float* k_lds = smem + DecLds<DK, DV>::k_off();
  float* ab_lds = smem + DecLds<DK, DV>::ab_off(W);
  float* y_lds = smem + DecLds<DK, DV>::y_off(W);
  float* c_lds = smem + DecLds<DK, DV>::c_off(W);
  float* v_lds = smem + DecLds<DK, DV>::v_off(W);
  float* dot_lds = smem + DecLds<DK, DV>::dot_off(W);

  const size_t qk_base = size_t(bh) * DK;
  const size_t v_base = size_t(bh) * DV;
  const size_t bufk_base = size_t(bh) * W * DK;
  const size_t bufv_base = size_t(bh) * W * DV;
  const size_t bufs_base = size_t(bh) * W;
  const float alpha_t = a.alpha[bh];
  const float beta_t = a.beta[bh];

  // Buffered keys of slots 0..f-1 (both paths), bounded so that lanes past
  // the fill fetch nothing.
  constexpr int KMAX = (64 * DK / 4 + NT - 1) / NT;
  const rsrc_t rk = make_rsrc(a.buf_k + bufk_base, uint32_t(f) * DK * 4);
  const rsrc_t ra = make_rsrc(a.buf_alpha + bufs_base, uint32_t(f) * 4);
  const rsrc_t rb = make_rsrc(a.buf_beta + bufs_base, uint32_t(f) * 4);
  float4 kt[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) kt[i] = bload_f4(rk, uint32_t(tid + i * NT) * 16);
  const float a_slot = bload_f1(ra, uint32_t(tid & 63) * 4);
  const float b_slot = bload_f1(rb, uint32_t(tid & 63) * 4);

  // current q, k in wave 0
  float qv[EK], kv[EK];
  if (wave == 0) {
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      qv[e] = load_in<IN_BF16>(a.q, qk_base + lane * EK + e);
      kv[e] = load_in<IN_BF16>(a.k, qk_base + lane * EK + e);
    }
  }

  if (!closing) {
    // ================================================================ open window
    constexpr int CPR = DK / 16;                  // 16-byte code chunks per row
    constexpr int NC = DV * DK / (16 * NT);       // chunks per thread
    constexpr int RG = DV / 4;                    // float4 row groups of v
    constexpr int NG = NT / RG;                   // slot groups
    constexpr int VMAX = (64 + NG - 1) / NG;
    static_assert(NC >= 1, "state too small for the tiling");

    const uint4* gc = reinterpret_cast<const uint4*>(a.codes + v_base * DK);
    uint4 cw[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) cw[i] = gc[tid + i * NT];

    const int rg = tid % RG;
    const int g = tid / RG;
    const rsrc_t rv = make_rsrc(a.buf_v + bufv_base, uint32_t(f) * DV * 4);
    float4 vt[VMAX];
#pragma unroll
    for (int i = 0; i < VMAX; ++i) vt[i] = bload_f4(rv, uint32_t((g + i * NG) * DV + rg * 4) * 4);
    float vcur = 0.f, srow = 0.f;
    if (tid < DV) {
      vcur = load_in<IN_BF16>(a.v, v_base + tid);
      srow = a.scales[v_base + tid];
    }

    // stage keys and slot scalars in LDS
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const int idx = tid + i * NT;
      if (idx < f * (DK / 4)) reinterpret_cast<float4*>(k_lds)[idx] = kt[i];
    }
    if (tid < 64) {
      ab_lds[tid] = a_slot;
      ab_lds[64 + tid] = b_slot;
    }
    if (wave == 0) {
      if constexpr (WHT) {
        fwht_group<EK, 64>(qv, lane);
        fwht_group<EK, 64>(kv, lane);
      }
    }
    __syncthreads();

    if (wave == 0) {
      // backward sweep: current write first, then buffered writes newest -> oldest
      float y[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) y[e] = qv[e];
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) part += kv[e] * y[e];
      float c = beta_t * wave_sum_uniform(part);
      if (lane == 0) c_lds[63] = c;
#pragma unroll
      for (int e = 0; e < EK; ++e) y[e] = alpha_t * (y[e] - c * kv[e]);
      for (int j = f - 1; j >= 0; --j) {
        float kj[EK];
#pragma unroll
        for (int e = 0; e < EK; ++e) kj[e] = k_lds[j * DK + lane * EK + e];
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) p += kj[e] * y[e];
        const float cj = ab_lds[64 + j] * wave_sum_uniform(p);
        if (lane == 0) c_lds[j] = cj;
        const float aj = ab_lds[j];
#pragma unroll
        for (int e = 0; e < EK; ++e) y[e] = aj * (y[e] - cj * kj[e]);
      }
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        y_lds[lane * EK + e] = y[e];
        a.buf_k[bufk_base + size_t(f) * DK + lane * EK + e] = kv[e];  // append k
      }
    }
    __syncthreads();

    // int8 rows . y  (row = chunk / CPR, 16 codes per chunk)
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int chunk = tid + i * NT;
      const int row = chunk / CPR;
      const int seg = chunk % CPR;
      const float4* y4 = reinterpret_cast<const float4*>(y_lds + seg * 16);
      const uint32_t w[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
      float p = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 yy = y4[q4];
        p += i8_at(w[q4], 0) * yy.x + i8_at(w[q4], 1) * yy.y + i8_at(w[q4], 2) * yy.z +
             i8_at(w[q4], 3) * yy.w;
      }
      p = group_sum<CPR>(p);
      if (seg == 0) dot_lds[row] = p;
    }
    // buffered values weighted by c_j
    {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < VMAX; ++i) {
        const int j = g + i * NG;
        const float cj = (j < f) ? c_lds[j] : 0.f;
        acc.x += cj * vt[i].x;
        acc.y += cj * vt[i].y;
        acc.z += cj * vt[i].z;
        acc.w += cj * vt[i].w;
      }
      reinterpret_cast<float4*>(v_lds + g * DV)[rg] = acc;
    }
    __syncthreads();

    if (tid < DV) {
      float vsum = 0.f;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) vsum += v_lds[gg * DV + tid];
      const float out = srow * dot_lds[tid] + vsum + c_lds[63] * vcur;
      store_out<OUT_BF16>(a.o, v_base + tid, out);
      a.buf_v[bufv_base + size_t(f) * DV + tid] = vcur;  // append v
    }
    if (tid == 0) {
      a.buf_alpha[bufs_base + f] = alpha_t;
      a.buf_beta[bufs_base + f] = beta_t;
      if (h == 0) a.fill_out[b] = f + 1;
    }
    return;
  }

  // ================================================================ window close
  constexpr int RW = DV / DEC_R;        // rows owned by this workgroup
  constexpr int LPR = NT / RW;          // lanes per row
  constexpr int CPL = DK / LPR;         // columns per lane
  constexpr int VCL = (64 * RW + NT - 1) / NT;
  static_assert(CPL >= 2 && CPL % 2 == 0, "close tiling");
  const int rr = tid / LPR;
  const int col0 = (tid % LPR) * CPL;
  const int row = r * RW + rr;

  // this workgroup's rows of the buffered values, all W-1 buffered slots
  const rsrc_t rv = make_rsrc(a.buf_v + bufv_base, uint32_t(W - 1) * DV * 4);
  float vb[VCL];
#pragma unroll
  for (int i = 0; i < VCL; ++i) {
    const int idx = tid + i * NT;
    vb[i] = bload_f1(rv, uint32_t((idx / RW) * DV + r * RW + idx % RW) * 4);
  }
  float vcur = 0.f;
  if (tid < RW) vcur = load_in<IN_BF16>(a.v, v_base + r * RW + tid);
  // dequantized rows in registers
  const float srow = a.scales[v_base + row];
  float s[CPL];
  {
    const int8_t* crow = a.codes + (v_base + row) * DK + col0;
    if constexpr (CPL == 8) {
      const uint2 w = *reinterpret_cast<const uint2*>(crow);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s[c] = i8_at(w.x, c) * srow;
        s[4 + c] = i8_at(w.y, c) * srow;
      }
    } else if constexpr (CPL == 4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(crow);
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] = i8_at(w, c) * srow;
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) s[c] = float(crow[c]) * srow;
    }
  }

#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const int idx = tid + i * NT;
    if (idx < f * (DK / 4)) reinterpret_cast<float4*>(k_lds)[idx] = kt[i];
  }
  if (tid < 64) {
    ab_lds[tid] = a_slot;
    ab_lds[64 + tid] = b_slot;
  }
#pragma unroll
  for (int i = 0; i < VCL; ++i) {
    const int idx = tid + i * NT;
    if (idx < (W - 1) * RW) v_lds[idx] = vb[i];
  }
  if (tid < RW) v_lds[(W - 1) * RW + tid] = vcur;
  __syncthreads();  // slot scalars are in place before wave 0 adds the current token's
  if (wave == 0) {
    if constexpr (WHT) {
      fwht_group<EK, 64>(qv, lane);
      fwht_group<EK, 64>(kv, lane);
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      k_lds[(W - 1) * DK + lane * EK + e] = kv[e];
      y_lds[lane * EK + e] = qv[e];
    }
    if (lane == 0) {
      ab_lds[W - 1] = alpha_t;
      ab_lds[64 + W - 1] = beta_t;
    }
  }
  __syncthreads();

  for (int j = 0; j < W; ++j) {
    float kj[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) kj[c] = k_lds[j * DK + col0 + c];
    float p = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) p += s[c] * kj[c];
    const float sk = group_sum<LPR>(p);
    const float aj = ab_lds[j];
    const float bj = ab_lds[64 + j];
    const float erase = bj * sk;
    const float write = bj * v_lds[j * RW + rr];
#pragma unroll
    for (int c = 0; c < CPL; ++c) s[c] = aj * (s[c] - erase * kj[c]) + write * kj[c];
  }

  float po = 0.f, amax = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    po += s[c] * y_lds[col0 + c];
    amax = fmaxf(amax, fabsf(s[c]));
  }
  po = group_sum<LPR>(po);
  amax = group_max<LPR>(amax);
  const float scale = codec_scale(amax);
  int8_t* crow = a.codes + (v_base + row) * DK + col0;
  if constexpr (CPL == 8) {
    uint2 w;
    w.x = pack4_i8(codec_code(s[0], scale), codec_code(s[1], scale), codec_code(s[2], scale),
                   codec_code(s[3], scale));
    w.y = pack4_i8(codec_code(s[4], scale), codec_code(s[5], scale), codec_code(s[6], scale),
                   codec_code(s[7], scale));
    *reinterpret_cast<uint2*>(crow) = w;
  } else if constexpr (CPL == 4) {
    *reinterpret_cast<uint32_t*>(crow) = pack4_i8(codec_code(s[0], scale), codec_code(s[1], scale),
                                                  codec_code(s[2], scale), codec_code(s[3], scale));
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) crow[c] = int8_t(codec_code(s[c], scale));
  }
  if ((tid % LPR) == 0) {
    a.scales[v_base + row] = scale;
    store_out<OUT_BF16>(a.o, v_base + row, po);
  }
  if (tid == 0 && r == 0 && h == 0) a.fill_out[b] = 0;
}

size_t decode_lds_bytes(int d_k, int d_v, int W) {
  const int RW = d_v / DEC_R;
  const int vsz = (4 * DEC_THREADS > W * RW) ? 4 * DEC_THREADS : W * RW;
  return sizeof(float) * size_t(W * d_k + 192 + d_k + vsz + d_v);
}

int decode_row_split() { return DEC_R; }

template <int DK, int DV, bool IB, bool OB, bool WHT>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const size_t lds = decode_lds_bytes(DK, DV, a.W);
  const unsigned grid = unsigned(a.B) * unsigned(a.H) * DEC_R;
  hipLaunchKernelGGL((decode_kernel<DK, DV, IB, OB, WHT>), dim3(grid), dim3(DEC_THREADS), lds, s,
                     a);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_dkdv(const DecodeArgs& a, bool ib, bool ob, bool wht, hipStream_t s) {
  if (ib) {
    if (ob) return wht ? launch_t<DK, DV, true, true, true>(a, s) : launch_t<DK, DV, true, true, false>(a, s);
    return wht ? launch_t<DK, DV, true, false, true>(a, s) : launch_t<DK, DV, true, false, false>(a, s);
  }
  if (ob) return wht ? launch_t<DK, DV, false, true, true>(a, s) : launch_t<DK, DV, false, true, false>(a, s);
  return wht ? launch_t<DK, DV, false, false, true>(a, s) : launch_t<DK, DV, false, false, false>(a, s);
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  DecodeArgs a{L.q,        L.k,        L.v,       L.alpha,   L.beta,   L.codes, L.scales, L.buf_k,
               L.buf_v,    L.buf_alpha, L.buf_beta, L.fill_in, L.fill_out, L.o,   L.B,      L.H,
               L.W};
  if (L.d_k == 128 && L.d_v == 128) return launch_dkdv<128, 128>(a, L.in_bf16, L.out_bf16, L.wht, stream);
  if (L.d_k == 128 && L.d_v == 64) return launch_dkdv<128, 64>(a, L.in_bf16, L.out_bf16, L.wht, stream);
  if (L.d_k == 64 && L.d_v == 128) return launch_dkdv<64, 128>(a, L.in_bf16, L.out_bf16, L.wht, stream);
  return launch_dkdv<64, 64>(a, L.in_bf16, L.out_bf16, L.wht, stream);
}

}  // namespace gdnq
