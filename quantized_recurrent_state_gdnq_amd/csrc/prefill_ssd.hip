// Chunkwise prefill of the scalar-decay SSD recurrence (Mamba-2 form)
//   S_t = a_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t,
// with q and k optionally rotated by the normalised Walsh-Hadamard matrix and
// quantized per token row to int8 codes + one fp32 scale ("LinQuant ...",
// abstract: SSD prefill with low-precision operands after a rotation;
// "Influence-Inspired Spectral Rotations ...", abstract: the Walsh-Hadamard
// rotation).  The state stays in fp32; it is never quantized.
//
// Chunk form (C = 64, g_i = sum_{s<=i} log a_s, e_i = exp(g_i),
// d_j = exp(g_C - g_j)), with q_i = sq_i cq_i and k_j = sk_j ck_j:
//   O[i]  = e_i sq_i (cq_i . S0) + sum_{j<=i} exp(g_i - g_j) sq_i sk_j (cq_i . ck_j) v_j
//   S_C   = e_C S0 + sum_j (d_j sk_j v_j) ck_j^T
// In plain bf16 mode cq, ck are q, k themselves and sq = sk = 1.
//
// Kernels:
//   operand -- (int8 mode) four lanes per token row of q or k: FWHT in
//              registers, row absmax, codec; codes and scales to the
//              workspace (one launch for both operands).
//   state   -- one workgroup per (sequence, head, 64 rows of d_v), the state
//              rows held in LDS as three bf16 parts (hi + mid + lo equals the
//              fp32 value exactly), three barriers per chunk.  All products on
//              bf16 MFMA: codes are exact in bf16; the state and the decayed,
//              scaled V are split into three parts, the output-only decay
//              matrix into two.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "mfma.h"

namespace gdnq {

namespace {

constexpr int SC = 64;    // chunk
constexpr int SDK = 128;  // d_k
constexpr int SRW = 64;   // state rows (of d_v) per workgroup

// ---------------------------------------------------------------- operand
// Four lanes per 128-element row (32 elements each): five butterfly stages
// inside the lane, the last two across the lane quad through DPP.
constexpr int OP_THREADS = 256;
constexpr int OP_LPR = 4;
constexpr int OP_E = SDK / OP_LPR;

struct OperandArgs {
  const uint16_t* x[2];  // q, k rows [rows][128] bf16
  int8_t* codes[2];      // [rows][128]
  float* scales[2];      // [rows]
  int64_t rows;
  bool wht;
};

__global__ __launch_bounds__(OP_THREADS) void ssd_operand_kernel(OperandArgs a) {
  const int op = blockIdx.y;
  const int tid = threadIdx.x;
  const int li = tid % OP_LPR;
  const int64_t row = int64_t(blockIdx.x) * (OP_THREADS / OP_LPR) + tid / OP_LPR;
  const bool valid = row < a.rows;
  float v[OP_E];
  const uint4* src = reinterpret_cast<const uint4*>(a.x[op] + row * SDK + li * OP_E);
#pragma unroll
  for (int p = 0; p < OP_E / 8; ++p) {
    const uint4 w = valid ? src[p] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * p + 2 * i] = bf16_lo(ww[i]);
      v[8 * p + 2 * i + 1] = bf16_hi(ww[i]);
    }
  }
  if (a.wht) {
    fwht_local<OP_E>(v);
    const bool up1 = (li & 1) != 0, up2 = (li & 2) != 0;
#pragma unroll
    for (int i = 0; i < OP_E; ++i) {
      const float o = dpp<DPP_XOR1>(v[i]);
      v[i] = up1 ? (o - v[i]) : (v[i] + o);
    }
#pragma unroll
    for (int i = 0; i < OP_E; ++i) {
      const float o = dpp<DPP_XOR2>(v[i]);
      v[i] = up2 ? (o - v[i]) : (v[i] + o);
    }
#pragma unroll
    for (int i = 0; i < OP_E; ++i) v[i] *= 0.08838834764831845f;  // 1/sqrt(128)
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < OP_E; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<OP_LPR>(amax);
  const float scale = codec_scale(amax);
  float cf[OP_E];
  codec_codes(v, scale, cf);
  if (!valid) return;
  uint4* dst = reinterpret_cast<uint4*>(a.codes[op] + row * SDK + li * OP_E);
#pragma unroll
  for (int p = 0; p < OP_E / 16; ++p) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack4_i8(int(cf[16 * p + 4 * i]), int(cf[16 * p + 4 * i + 1]), int(cf[16 * p + 4 * i + 2]),
                      int(cf[16 * p + 4 * i + 3]));
    dst[p] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (li == 0) a.scales[op][row] = scale;
}

// ---------------------------------------------------------------- state pass
struct SsdArgs {
  const void* q;       // int8 codes [B,T,H,128] or bf16 [B,T,H,128]
  const void* k;
  const float* sq;     // [B,T,H] (int8 mode)
  const float* sk;
  const uint16_t* v;   // [B,T,H,d_v] bf16
  const float* alpha;  // [B,T,H]
  void* o;             // [B,T,H,d_v]
  float* state;        // [B,H,d_v,128]
  int B, T, H, DV;
};

constexpr int QP = 136;  // bf16 pitch of [64][128] (codes of q, k; state parts)
constexpr int JP = 72;   // bf16 pitch of [64][64] planes (M parts, V^T, W parts)

constexpr int OFF_Q = 0;                         // q codes [64][QP] bf16
constexpr int OFF_K = OFF_Q + SC * QP * 2;       // k codes [64][QP] bf16
constexpr int OFF_KT = OFF_K + SC * QP * 2;      // k codes transposed [128][64], xor-swizzled granules
constexpr int OFF_S = OFF_KT + SDK * SC * 2;     // state hi/mid/lo [3][64][QP] bf16
constexpr int OFF_M = OFF_S + 3 * SRW * QP * 2;  // M hi/lo [2][64][JP] bf16
constexpr int OFF_V = OFF_M + 2 * SC * JP * 2;   // V^T [64 rows][JP] bf16
constexpr int OFF_W = OFF_V + SRW * JP * 2;      // (V o d o sk)^T hi/mid/lo [3][64][JP] bf16
constexpr int OFF_F = OFF_W + 3 * SRW * JP * 2;  // g, exp(g), exp(g_C - g), sq, sk [5][64]
constexpr int SSD_LDS = OFF_F + 5 * SC * 4;
static_assert(SSD_LDS <= 160 * 1024, "SSD LDS");

__device__ __forceinline__ int kt_at(int d, int j) {
  return d * SC + ((((j >> 3) ^ (d >> 3)) & 7) << 3) + (j & 7);
}

__device__ __forceinline__ void tile_lower(int tt, int& it, int& jt) {
  it = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
  jt = tt - it * (it + 1) / 2;
}

__device__ __forceinline__ float exp_dec(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ uint2 u2_of(const bf16x4& v) { return __builtin_bit_cast(uint2, v); }

__device__ __forceinline__ bf16x8 u4_bf16(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// 8 int8 codes (two words) -> 8 bf16 packed in a uint4
__device__ __forceinline__ uint4 i8x8_bf16_u4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(uint4, i8x8_to_bf16(make_uint2(lo, hi)));
}

template <bool I8, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void ssd_state_kernel(SsdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __bf16* Qc = reinterpret_cast<__bf16*>(lds + OFF_Q);
  __bf16* Kc = reinterpret_cast<__bf16*>(lds + OFF_K);
  __bf16* KT = reinterpret_cast<__bf16*>(lds + OFF_KT);
  __bf16* Sp = reinterpret_cast<__bf16*>(lds + OFF_S);
  __bf16* Mp = reinterpret_cast<__bf16*>(lds + OFF_M);
  __bf16* Vt = reinterpret_cast<__bf16*>(lds + OFF_V);
  __bf16* Wp = reinterpret_cast<__bf16*>(lds + OFF_W);
  float* gl = reinterpret_cast<float*>(lds + OFF_F);
  float* el = gl + SC;
  float* dl = el + SC;
  float* sql = dl + SC;
  float* skl = sql + SC;

  const int nrb = a.DV / SRW;
  const int chain = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int b = chain / a.H, h = chain % a.H;
  const int r0 = rb * SRW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int NC = a.T / SC;
  const size_t tokb = size_t(b) * a.T;
  const size_t HK = size_t(a.H) * SDK, HV = size_t(a.H) * a.DV;

  // load mapping: token pair jp, 8 dims (k, q) or 4 rows (v) per group g16
  const int jp = tid & 31, g16 = tid >> 5;
  const size_t kq0 = (tokb + 2 * jp) * HK + size_t(h) * SDK + 8 * g16;  // element offset, chunk 0
  const size_t v0 = (tokb + 2 * jp) * HV + size_t(h) * a.DV + r0 + 4 * g16;
  const size_t chunk_kq = SC * HK, chunk_v = SC * HV;

  // prefetched next chunk: q, k as two 8-element pieces (tokens 2 jp, 2 jp + 1),
  // v as two 4-row pieces, and per-token alpha, sq, sk (threads < 64)
  uint4 qa, qb, ka, kb;
  uint2 va, vb;
  float av = 1.f, sqv = 1.f, skv = 1.f;
  auto load = [&](int c) {
    const size_t o = kq0 + size_t(c) * chunk_kq;
    if constexpr (I8) {
      const int8_t* qp = static_cast<const int8_t*>(a.q) + o;
      const int8_t* kp = static_cast<const int8_t*>(a.k) + o;
      const uint2 q0 = *reinterpret_cast<const uint2*>(qp), q1 = *reinterpret_cast<const uint2*>(qp + HK);
      const uint2 k0 = *reinterpret_cast<const uint2*>(kp), k1 = *reinterpret_cast<const uint2*>(kp + HK);
      qa = make_uint4(q0.x, q0.y, 0u, 0u);
      qb = make_uint4(q1.x, q1.y, 0u, 0u);
      ka = make_uint4(k0.x, k0.y, 0u, 0u);
      kb = make_uint4(k1.x, k1.y, 0u, 0u);
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + o;
      const uint16_t* kp = static_cast<const uint16_t*>(a.k) + o;
      qa = *reinterpret_cast<const uint4*>(qp);
      qb = *reinterpret_cast<const uint4*>(qp + HK);
      ka = *reinterpret_cast<const uint4*>(kp);
      kb = *reinterpret_cast<const uint4*>(kp + HK);
    }
    const uint16_t* vp = a.v + v0 + size_t(c) * chunk_v;
    va = *reinterpret_cast<const uint2*>(vp);
    vb = *reinterpret_cast<const uint2*>(vp + HV);
    if (tid < 64) {
      const size_t t = (tokb + size_t(c) * SC + tid) * a.H + h;
      av = a.alpha[t];
      if constexpr (I8) {
        sqv = a.sq[t];
        skv = a.sk[t];
      }
    }
  };
  auto stage = [&]() {
    uint4 q0 = qa, q1 = qb, k0 = ka, k1 = kb;
    if constexpr (I8) {
      q0 = i8x8_bf16_u4(qa.x, qa.y);
      q1 = i8x8_bf16_u4(qb.x, qb.y);
      k0 = i8x8_bf16_u4(ka.x, ka.y);
      k1 = i8x8_bf16_u4(kb.x, kb.y);
    }
    *reinterpret_cast<uint4*>(Qc + (2 * jp) * QP + 8 * g16) = q0;
    *reinterpret_cast<uint4*>(Qc + (2 * jp + 1) * QP + 8 * g16) = q1;
    *reinterpret_cast<uint4*>(Kc + (2 * jp) * QP + 8 * g16) = k0;
    *reinterpret_cast<uint4*>(Kc + (2 * jp + 1) * QP + 8 * g16) = k1;
    {  // k^T: one dword = tokens (2 jp, 2 jp + 1) of dim 8 g16 + e
      const uint32_t w0[4] = {k0.x, k0.y, k0.z, k0.w};
      const uint32_t w1[4] = {k1.x, k1.y, k1.z, k1.w};
      uint32_t* kt = reinterpret_cast<uint32_t*>(KT);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        kt[kt_at(8 * g16 + e, 2 * jp) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      }
    }
    {  // V^T: rows 4 g16 + e, tokens (2 jp, 2 jp + 1)
      const uint32_t w0[2] = {va.x, va.y}, w1[2] = {vb.x, vb.y};
      uint32_t* vt = reinterpret_cast<uint32_t*>(Vt);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        vt[((4 * g16 + e) * JP + 2 * jp) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      }
    }
    if (tid < 64) {  // g = inclusive prefix sum of log a over the chunk
      float g = logf(av);
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const float o = __shfl_up(g, s, 64);
        if (lane >= s) g += o;
      }
      const float gC = __shfl(g, 63, 64);
      gl[tid] = g;
      el[tid] = expf(g);
      dl[tid] = expf(gC - g);
      sql[tid] = sqv;
      skl[tid] = skv;
    }
  };

  // zero initial state
  for (int e = tid; e < 3 * SRW * QP / 8; e += 512) reinterpret_cast<uint4*>(Sp)[e] = make_uint4(0u, 0u, 0u, 0u);
  if (NC > 0) {
    load(0);
    stage();
    if (NC > 1) load(1);
  }
  __syncthreads();

  const int it = wave >> 1, rp = (wave & 1) * 2;  // token tile, first of two row tiles (O, Q S0^T)
  const int nks = (it >> 1) + 1;
  const int i0 = it * 16 + 4 * lq;

  for (int c = 0; c < NC; ++c) {
    const size_t tok0 = tokb + size_t(c) * SC;
    // ---- A: Q S0^T (state in three parts), M = L o (sq sk Q K^T), W = (V o d o sk)^T
    float os[2][4];
    {
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        const bf16x8 aq = lds_bf16x8(Qc + (it * 16 + lr) * QP + kk);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const __bf16* sp = Sp + ((rp + t) * 16 + lr) * QP + kk;
          acc[t] = mfma16(aq, lds_bf16x8(sp + 2 * SRW * QP), acc[t]);
          acc[t] = mfma16(aq, lds_bf16x8(sp + SRW * QP), acc[t]);
          acc[t] = mfma16(aq, lds_bf16x8(sp), acc[t]);
        }
      }
      const float4 e4 = *reinterpret_cast<const float4*>(el + i0);
      const float4 s4 = *reinterpret_cast<const float4*>(sql + i0);
      const float es[4] = {e4.x * s4.x, e4.y * s4.y, e4.z * s4.z, e4.w * s4.w};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) os[t][q] = es[q] * acc[t][q];
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int tt = wave + 8 * n;
      if (tt < 12) {
        int mi, mj;
        float m4[4] = {0.f, 0.f, 0.f, 0.f};
        if (tt < 10) {  // M^T tile D[j][i] = ck_j . cq_i
          tile_lower(tt, mi, mj);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int kk = ks * 32 + 8 * lq;
            acc = mfma16(lds_bf16x8(Kc + (mj * 16 + lr) * QP + kk), lds_bf16x8(Qc + (mi * 16 + lr) * QP + kk), acc);
          }
          const int i = mi * 16 + lr;
          const float gi = gl[i], si = sql[i];
          const float4 g4 = *reinterpret_cast<const float4*>(gl + mj * 16 + 4 * lq);
          const float4 k4 = *reinterpret_cast<const float4*>(skl + mj * 16 + 4 * lq);
          const float gj[4] = {g4.x, g4.y, g4.z, g4.w}, sj[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = mj * 16 + 4 * lq + q;
            m4[q] = (j <= i) ? exp_dec(gi - gj[q]) * (si * sj[q]) * acc[q] : 0.f;
          }
        } else {  // zero tiles above the diagonal reached by the 32-token steps
          mi = tt == 10 ? 0 : 2;
          mj = mi + 1;
        }
        bf16x4 h1, h2;
        split2(m4, h1, h2);
        const int i = mi * 16 + lr, j0 = mj * 16 + 4 * lq;
        *reinterpret_cast<uint2*>(Mp + i * JP + j0) = u2_of(h1);
        *reinterpret_cast<uint2*>(Mp + SC * JP + i * JP + j0) = u2_of(h2);
      }
    }
    {  // W[r][j] = V[j][r] d_j sk_j: row tid / 8, tokens [8 (tid % 8), +8)
      const int rr = tid >> 3, j0 = (tid & 7) * 8;
      const bf16x8 vv = lds_bf16x8(Vt + rr * JP + j0);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = float(vv[e]) * (dl[j0 + e] * skl[j0 + e]);
      bf16x8 h1, h2, h3;
      split3(x, h1, h2, h3);
      *reinterpret_cast<bf16x8*>(Wp + rr * JP + j0) = h1;
      *reinterpret_cast<bf16x8*>(Wp + SRW * JP + rr * JP + j0) = h2;
      *reinterpret_cast<bf16x8*>(Wp + 2 * SRW * JP + rr * JP + j0) = h3;
    }
    __syncthreads();

    // ---- B: O = base + M V (V exact), and S_C^T = e_C S0^T + K^T W
    {
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      for (int ks = 0; ks < nks; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        const bf16x8 m1 = lds_bf16x8(Mp + (it * 16 + lr) * JP + kk);
        const bf16x8 m2 = lds_bf16x8(Mp + SC * JP + (it * 16 + lr) * JP + kk);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 vv = lds_bf16x8(Vt + ((rp + t) * 16 + lr) * JP + kk);
          acc[t] = mfma16(m2, vv, acc[t]);
          acc[t] = mfma16(m1, vv, acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = (rp + t) * 16 + lr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const size_t oi = (tok0 + i0 + q) * HV + size_t(h) * a.DV + r0 + r;
          const float ov = os[t][q] + acc[t][q];
          if constexpr (OUT_BF16) static_cast<uint16_t*>(a.o)[oi] = uint16_t(f32_to_bf16_bits(ov));
          else static_cast<float*>(a.o)[oi] = ov;
        }
      }
    }
    {
      const int rt = wave & 3, dt0 = (wave >> 2) * 4;  // row tile, four dim tiles
      const int r = rt * 16 + lr;
      bf16x8 w1[2], w2[2], w3[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* wp = Wp + r * JP + ks * 32 + 8 * lq;
        w1[ks] = lds_bf16x8(wp);
        w2[ks] = lds_bf16x8(wp + SRW * JP);
        w3[ks] = lds_bf16x8(wp + 2 * SRW * JP);
      }
      const float eC = el[SC - 1];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int dt = dt0 + t;
        const int d0 = dt * 16 + 4 * lq;
        __bf16* sp = Sp + r * QP + d0;
        const bf16x4 p1 = *reinterpret_cast<const bf16x4*>(sp);
        const bf16x4 p2 = *reinterpret_cast<const bf16x4*>(sp + SRW * QP);
        const bf16x4 p3 = *reinterpret_cast<const bf16x4*>(sp + 2 * SRW * QP);
        f32x4 acc;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = eC * ((float(p1[q]) + float(p2[q])) + float(p3[q]));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 ak = lds_bf16x8(KT + kt_at(dt * 16 + lr, ks * 32 + 8 * lq));
          acc = mfma16(ak, w3[ks], acc);
          acc = mfma16(ak, w2[ks], acc);
          acc = mfma16(ak, w1[ks], acc);
        }
        const float x[4] = {acc[0], acc[1], acc[2], acc[3]};
        bf16x4 h1, h2, h3;
        split3(x, h1, h2, h3);
        *reinterpret_cast<uint2*>(sp) = u2_of(h1);
        *reinterpret_cast<uint2*>(sp + SRW * QP) = u2_of(h2);
        *reinterpret_cast<uint2*>(sp + 2 * SRW * QP) = u2_of(h3);
      }
    }
    __syncthreads();

    // ---- C: stage the next chunk, prefetch the one after
    if (c + 1 < NC) {
      stage();
      if (c + 2 < NC) load(c + 2);
    }
    __syncthreads();
  }

  {  // final state (rows r0.., all 128 dims): hi + mid + lo
    float* dst = a.state + ((size_t(b) * a.H + h) * a.DV + r0) * SDK;
    for (int e = tid; e < SRW * SDK / 4; e += 512) {
      const int rr = e / (SDK / 4), d0 = (e % (SDK / 4)) * 4;
      const __bf16* sp = Sp + rr * QP + d0;
      const bf16x4 p1 = *reinterpret_cast<const bf16x4*>(sp);
      const bf16x4 p2 = *reinterpret_cast<const bf16x4*>(sp + SRW * QP);
      const bf16x4 p3 = *reinterpret_cast<const bf16x4*>(sp + 2 * SRW * QP);
      float4 s;
      s.x = (float(p1[0]) + float(p2[0])) + float(p3[0]);
      s.y = (float(p1[1]) + float(p2[1])) + float(p3[1]);
      s.z = (float(p1[2]) + float(p2[2])) + float(p3[2]);
      s.w = (float(p1[3]) + float(p2[3])) + float(p3[3]);
      *reinterpret_cast<float4*>(dst + size_t(rr) * SDK + d0) = s;
    }
  }
}

size_t ssd_rows(const PrefillLaunch& L) { return size_t(L.B) * L.T * L.H; }

}  // namespace

size_t prefill_ssd_workspace_bytes(const PrefillLaunch& L) {
  if (!L.int8_qk) return 0;
  const size_t rows = ssd_rows(L);
  return 2 * rows * SDK + 2 * rows * 4;  // q codes, k codes, q scales, k scales
}

hipError_t launch_prefill_ssd(const PrefillLaunch& L, hipStream_t stream) {
  const size_t rows = ssd_rows(L);
  const void* qsrc = L.q;
  const void* ksrc = L.k;
  const float* sq = nullptr;
  const float* sk = nullptr;
  if (L.int8_qk && rows > 0) {
    int8_t* cq = static_cast<int8_t*>(L.workspace);
    int8_t* ck = cq + rows * SDK;
    float* fq = reinterpret_cast<float*>(ck + rows * SDK);
    float* fk = fq + rows;
    const unsigned grid = unsigned((rows + OP_THREADS / OP_LPR - 1) / (OP_THREADS / OP_LPR));
    OperandArgs oa{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k)}, {cq, ck}, {fq, fk},
                   int64_t(rows), L.wht};
    hipLaunchKernelGGL(ssd_operand_kernel, dim3(grid, 2), dim3(OP_THREADS), 0, stream, oa);
    if (hipError_t e = hipGetLastError()) return e;
    qsrc = cq;
    ksrc = ck;
    sq = fq;
    sk = fk;
  }
  SsdArgs s{qsrc, ksrc, sq, sk, static_cast<const uint16_t*>(L.v), L.alpha, L.o, L.state_f32,
            L.B, L.T, L.H, L.d_v};
  const unsigned grid = unsigned(L.B) * L.H * (L.d_v / SRW);
  void (*kern)(SsdArgs) = L.int8_qk ? (L.out_bf16 ? &ssd_state_kernel<true, true> : &ssd_state_kernel<true, false>)
                                    : (L.out_bf16 ? &ssd_state_kernel<false, true> : &ssd_state_kernel<false, false>);
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, SSD_LDS))
    return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), SSD_LDS, stream, s);
  return hipGetLastError();
}

}  // namespace gdnq
