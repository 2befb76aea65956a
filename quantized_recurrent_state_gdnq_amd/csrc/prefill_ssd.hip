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
//   state   -- one workgroup per (sequence, head, 64 rows of d_v), two
//              barriers per chunk.  Four state waves hold 16 rows each of the
//              fp32 state as MFMA accumulators (eight 16x16 tiles of S^T) and
//              update them in place; four aux waves build the decay matrix,
//              form the output and stage the next chunk.  All products on
//              bf16 MFMA: codes are exact in bf16; the state and the decayed,
//              scaled V are split into three bf16 parts (hi + mid + lo equals
//              the fp32 value exactly), the output-only decay matrix into two.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include <type_traits>

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

constexpr int QP = 136;   // bf16 pitch of [64][128] (codes of q, k)
constexpr int JP = 72;    // bf16 pitch of [64][64] planes (M parts, V^T, W parts)

constexpr int OFF_Q = 0;                          // q codes [64][QP] bf16
constexpr int OFF_K = OFF_Q + SC * QP * 2;        // k codes [64][QP] bf16
constexpr int OFF_KT = OFF_K + SC * QP * 2;       // [2] k codes transposed [128][64], xor-swizzled granules
constexpr int OFF_M = OFF_KT + 2 * SDK * SC * 2;  // M hi/lo [2][64][JP] bf16
constexpr int OFF_V = OFF_M + 2 * SC * JP * 2;    // [2] V^T [64 rows][JP] bf16
constexpr int OFF_W = OFF_V + 2 * SRW * JP * 2;   // (V o d o sk)^T hi/mid/lo [3][64][JP] bf16
constexpr int OFF_QS = OFF_W + 3 * SRW * JP * 2;  // Q S0^T tiles [4 it][4 rt][64 lanes] float4
constexpr int OFF_F = OFF_QS + SC * SRW * 4;      // [2] g, exp(g), exp(g_C - g), sq, sk [5][64]
constexpr int SSD_LDS = OFF_F + 2 * 5 * SC * 4;
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

// 8 int8 codes (two words) -> 8 bf16 packed in a uint4
__device__ __forceinline__ uint4 i8x8_bf16_u4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(uint4, i8x8_to_bf16(make_uint2(lo, hi)));
}

// Per workgroup (sequence, head, 64 rows of d_v), eight waves:
//   state waves 0..3 hold rows 16 rt .. +16 of the state, all 128 columns,
//   as fp32 accumulators S^T[d][r] (eight 16x16 tiles in the MFMA output
//   layout; two adjacent tiles form a B operand of the 16x16x32 product
//   under a k order both operands share, so Q S0^T reads the state straight
//   from registers, in three bf16 parts), and build W = (V o d o sk)^T;
//   aux waves 4..7 build M = L o (sq sk Q K^T), produce the output rows of
//   token tile it, stage the next chunk and prefetch the one after.
// Two barriers per chunk:
//   A  state: Q S0^T -> LDS, W            | aux: M
//   B  state: S^T = e_C S^T + K^T W       | aux: O = e sq (Q S0^T) + M V; stage c+1, load c+2
template <bool I8, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void ssd_state_kernel(SsdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __bf16* Qc = reinterpret_cast<__bf16*>(lds + OFF_Q);
  __bf16* Kc = reinterpret_cast<__bf16*>(lds + OFF_K);
  __bf16* KTb = reinterpret_cast<__bf16*>(lds + OFF_KT);
  __bf16* Mp = reinterpret_cast<__bf16*>(lds + OFF_M);
  __bf16* Vtb = reinterpret_cast<__bf16*>(lds + OFF_V);
  __bf16* Wp = reinterpret_cast<__bf16*>(lds + OFF_W);
  float4* QSl = reinterpret_cast<float4*>(lds + OFF_QS);
  float* Fb = reinterpret_cast<float*>(lds + OFF_F);

  const int nrb = a.DV / SRW;
  const int chain = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int b = chain / a.H, h = chain % a.H;
  const int r0 = rb * SRW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int NC = a.T / SC;
  const size_t tokb = size_t(b) * a.T;
  const size_t HK = size_t(a.H) * SDK, HV = size_t(a.H) * a.DV;
  const bool state_wave = wave < 4;
  const int rt = wave & 3;        // state waves: row tile
  const int it = wave & 3;        // aux waves: token tile
  const int at = tid & 255;       // aux thread index

  // ---- prefetch (aux threads): k as token pair jp, 16 dims 16 g8 .. ; q as
  // token at / 4, 32 dims; v as token pair jp, 8 rows 8 g8 ..; scalars (at < 64)
  const int jp = at & 31, g8 = at >> 5;
  const int qt = at >> 2, qd = (at & 3) * 32;
  uint4 ka[2], kb[2], qw[4], va, vb;
  float av = 1.f, sqv = 1.f, skv = 1.f;
  auto load = [&](int c) __attribute__((always_inline)) {
    const size_t t0 = tokb + size_t(c) * SC;
    const size_t ko = (t0 + 2 * jp) * HK + size_t(h) * SDK + 16 * g8;
    const size_t qo = (t0 + qt) * HK + size_t(h) * SDK + qd;
    if constexpr (I8) {
      const int8_t* kp = static_cast<const int8_t*>(a.k) + ko;
      const int8_t* qp = static_cast<const int8_t*>(a.q) + qo;
      ka[0] = *reinterpret_cast<const uint4*>(kp);
      kb[0] = *reinterpret_cast<const uint4*>(kp + HK);
      qw[0] = *reinterpret_cast<const uint4*>(qp);
      qw[1] = *reinterpret_cast<const uint4*>(qp + 16);
    } else {
      const uint16_t* kp = static_cast<const uint16_t*>(a.k) + ko;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qo;
      ka[0] = *reinterpret_cast<const uint4*>(kp);
      ka[1] = *reinterpret_cast<const uint4*>(kp + 8);
      kb[0] = *reinterpret_cast<const uint4*>(kp + HK);
      kb[1] = *reinterpret_cast<const uint4*>(kp + HK + 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) qw[e] = *reinterpret_cast<const uint4*>(qp + 8 * e);
    }
    const uint16_t* vp = a.v + (t0 + 2 * jp) * HV + size_t(h) * a.DV + r0 + 8 * g8;
    va = *reinterpret_cast<const uint4*>(vp);
    vb = *reinterpret_cast<const uint4*>(vp + HV);
    {  // every aux lane loads, so each load is issued on every path; lanes at < 64 keep them
      const size_t t = (t0 + (at & 63)) * a.H + h;
      av = a.alpha[t];
      if constexpr (I8) {
        sqv = a.sq[t];
        skv = a.sk[t];
      }
    }
  };
  auto stage = [&](int par) __attribute__((always_inline)) {
    uint4 k0[2], k1[2], q8[4];
    if constexpr (I8) {
      k0[0] = i8x8_bf16_u4(ka[0].x, ka[0].y);
      k0[1] = i8x8_bf16_u4(ka[0].z, ka[0].w);
      k1[0] = i8x8_bf16_u4(kb[0].x, kb[0].y);
      k1[1] = i8x8_bf16_u4(kb[0].z, kb[0].w);
      q8[0] = i8x8_bf16_u4(qw[0].x, qw[0].y);
      q8[1] = i8x8_bf16_u4(qw[0].z, qw[0].w);
      q8[2] = i8x8_bf16_u4(qw[1].x, qw[1].y);
      q8[3] = i8x8_bf16_u4(qw[1].z, qw[1].w);
    } else {
      k0[0] = ka[0];
      k0[1] = ka[1];
      k1[0] = kb[0];
      k1[1] = kb[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) q8[e] = qw[e];
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      *reinterpret_cast<uint4*>(Kc + (2 * jp) * QP + 16 * g8 + 8 * e) = k0[e];
      *reinterpret_cast<uint4*>(Kc + (2 * jp + 1) * QP + 16 * g8 + 8 * e) = k1[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(Qc + qt * QP + qd + 8 * e) = q8[e];
    {  // k^T: dword = tokens (2 jp, 2 jp + 1) of dim 16 g8 + e
      uint32_t* kt = reinterpret_cast<uint32_t*>(KTb + par * SDK * SC);
      const uint32_t w0[8] = {k0[0].x, k0[0].y, k0[0].z, k0[0].w, k0[1].x, k0[1].y, k0[1].z, k0[1].w};
      const uint32_t w1[8] = {k1[0].x, k1[0].y, k1[0].z, k1[0].w, k1[1].x, k1[1].y, k1[1].z, k1[1].w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        kt[kt_at(16 * g8 + e, 2 * jp) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      }
    }
    {  // V^T: rows 8 g8 + e, tokens (2 jp, 2 jp + 1)
      uint32_t* vt = reinterpret_cast<uint32_t*>(Vtb + par * SRW * JP);
      const uint32_t w0[4] = {va.x, va.y, va.z, va.w}, w1[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        vt[((8 * g8 + e) * JP + 2 * jp) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      }
    }
    if (wave == 4) {  // g = inclusive prefix sum of log a over the chunk (lane = token)
      const float g = wave_scan_incl(logf(av));
      const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 63));
      float* F = Fb + par * 5 * SC;
      F[lane] = g;
      F[SC + lane] = expf(g);
      F[2 * SC + lane] = expf(gC - g);
      F[3 * SC + lane] = sqv;
      F[4 * SC + lane] = skv;
    }
  };

  // The two roles run separate loops (same barrier count per chunk), so each
  // gets its own register allocation: the prefetch registers of the aux
  // waves never have to survive the state waves' code
  if (state_wave) {
    f32x4 S[8];  // S^T tiles
#pragma unroll
    for (int d = 0; d < 8; ++d) S[d] = {0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int c = 0; c < NC; ++c) {
      const int par = c & 1;
      const float* F = Fb + par * 5 * SC;
      const __bf16* KT = KTb + par * SDK * SC;
      const __bf16* Vt = Vtb + par * SRW * JP;
      // -------------------------------------------------------------- A
      // Q S0^T for the four token tiles of row tile rt, 32 dims per product:
      // the k slots of lane group lq are dims 32 m + 4 lq + {0..3} (tile 2m)
      // and 32 m + 16 + 4 lq + {0..3} (tile 2m + 1), the same order in both
      // operands, so the state tiles feed the B operand as they are
      auto q_ops = [&](int m, bf16x8* aq) __attribute__((always_inline)) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const __bf16* qr = Qc + (ti * 16 + lr) * QP + 32 * m + 4 * lq;
          const uint2 lo = *reinterpret_cast<const uint2*>(qr);
          const uint2 hi = *reinterpret_cast<const uint2*>(qr + 16);
          aq[ti] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
      };
      f32x4 acc[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) acc[ti] = {0.f, 0.f, 0.f, 0.f};
      bf16x8 aq[2][4];
      q_ops(0, aq[0]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < 3) q_ops(m + 1, aq[(m + 1) & 1]);
        const float x[8] = {S[2 * m][0], S[2 * m][1], S[2 * m][2], S[2 * m][3],
                            S[2 * m + 1][0], S[2 * m + 1][1], S[2 * m + 1][2], S[2 * m + 1][3]};
        bf16x8 bp[3];
        split3(x, bp[0], bp[1], bp[2]);
#pragma unroll
        for (int p = 2; p >= 0; --p)
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) acc[ti] = mfma16(aq[m & 1][ti], bp[p], acc[ti]);
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        QSl[(ti * 4 + rt) * 64 + lane] = make_float4(acc[ti][0], acc[ti][1], acc[ti][2], acc[ti][3]);
      {  // W[r][j] = V[j][r] d_j sk_j for this row tile: row 16 rt + lane / 4, tokens [16 (lane % 4), +16)
        const int rr = rt * 16 + (lane >> 2), j0 = (lane & 3) * 16;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int jb = j0 + 8 * hh;
          const bf16x8 vv = lds_bf16x8(Vt + rr * JP + jb);
          const float4 d0 = *reinterpret_cast<const float4*>(F + 2 * SC + jb);
          const float4 d1 = *reinterpret_cast<const float4*>(F + 2 * SC + jb + 4);
          const float4 k0 = *reinterpret_cast<const float4*>(F + 4 * SC + jb);
          const float4 k1 = *reinterpret_cast<const float4*>(F + 4 * SC + jb + 4);
          const float dk[8] = {d0.x * k0.x, d0.y * k0.y, d0.z * k0.z, d0.w * k0.w,
                               d1.x * k1.x, d1.y * k1.y, d1.z * k1.z, d1.w * k1.w};
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = float(vv[e]) * dk[e];
          bf16x8 w1, w2, w3;
          split3(x, w1, w2, w3);
          *reinterpret_cast<bf16x8*>(Wp + rr * JP + jb) = w1;
          *reinterpret_cast<bf16x8*>(Wp + SRW * JP + rr * JP + jb) = w2;
          *reinterpret_cast<bf16x8*>(Wp + 2 * SRW * JP + rr * JP + jb) = w3;
        }
      }
      __syncthreads();
      // -------------------------------------------------------------- B
      const float eC = F[SC + SC - 1];
      bf16x8 w1[2], w2[2], w3[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* wp = Wp + (rt * 16 + lr) * JP + ks * 32 + 8 * lq;
        w1[ks] = lds_bf16x8(wp);
        w2[ks] = lds_bf16x8(wp + SRW * JP);
        w3[ks] = lds_bf16x8(wp + 2 * SRW * JP);
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        f32x4 acc = S[d];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] *= eC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 ak = lds_bf16x8(KT + kt_at(d * 16 + lr, ks * 32 + 8 * lq));
          acc = mfma16(ak, w3[ks], acc);
          acc = mfma16(ak, w2[ks], acc);
          acc = mfma16(ak, w1[ks], acc);
        }
        S[d] = acc;
      }
      __syncthreads();
    }
    // final state rows r0 + 16 rt + lr, columns d: S^T tile layout
    float* dst = a.state + ((size_t(b) * a.H + h) * a.DV + r0 + rt * 16 + lr) * SDK;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<float4*>(dst + d * 16 + 4 * lq) = make_float4(S[d][0], S[d][1], S[d][2], S[d][3]);
  } else {
    if (NC > 0) {
      load(0);
      stage(0);
      load(NC > 1 ? 1 : 0);
    }
    __syncthreads();
    for (int c = 0; c < NC; ++c) {
      const int par = c & 1;
      const float* F = Fb + par * 5 * SC;
      const __bf16* Vt = Vtb + par * SRW * JP;
      // -------------------------------------------------------------- A
      // M tiles, spread over the four aux waves: the ten lower tiles, then
      // the two zero tiles above the diagonal that the 32-token steps reach
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        const int tt = it + 4 * n;
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
          const float gi = F[i], si = F[3 * SC + i];
          const float4 g4 = *reinterpret_cast<const float4*>(F + mj * 16 + 4 * lq);
          const float4 k4 = *reinterpret_cast<const float4*>(F + 4 * SC + mj * 16 + 4 * lq);
          const float gj[4] = {g4.x, g4.y, g4.z, g4.w}, sj[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = mj * 16 + 4 * lq + q;
            m4[q] = (j <= i) ? exp_dec(gi - gj[q]) * (si * sj[q]) * acc[q] : 0.f;
          }
        } else {
          mi = tt == 10 ? 0 : 2;
          mj = mi + 1;
        }
        bf16x4 h1, h2;
        split2(m4, h1, h2);
        const int i = mi * 16 + lr, j0 = mj * 16 + 4 * lq;
        *reinterpret_cast<uint2*>(Mp + i * JP + j0) = u2_of(h1);
        *reinterpret_cast<uint2*>(Mp + SC * JP + i * JP + j0) = u2_of(h2);
      }
      __syncthreads();
      // -------------------------------------------------------------- B
      const size_t tok0 = tokb + size_t(c) * SC;
      const int i0 = it * 16 + 4 * lq;
      const float4 e4 = *reinterpret_cast<const float4*>(F + SC + i0);
      const float4 q4 = *reinterpret_cast<const float4*>(F + 3 * SC + i0);
      const float es[4] = {e4.x * q4.x, e4.y * q4.y, e4.z * q4.z, e4.w * q4.w};
      f32x4 mv[4];  // (M V) for the four row tiles
      auto mv_tiles = [&](auto nk) __attribute__((always_inline)) {
        constexpr int NK = decltype(nk)::value;
        bf16x8 m1[NK], m2[NK];
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const int kk = ks * 32 + 8 * lq;
          m1[ks] = lds_bf16x8(Mp + (it * 16 + lr) * JP + kk);
          m2[ks] = lds_bf16x8(Mp + SC * JP + (it * 16 + lr) * JP + kk);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            const bf16x8 vv = lds_bf16x8(Vt + (rr * 16 + lr) * JP + ks * 32 + 8 * lq);
            acc = mfma16(m2[ks], vv, acc);
            acc = mfma16(m1[ks], vv, acc);
          }
          mv[rr] = acc;
        }
      };
      if (it < 2) mv_tiles(std::integral_constant<int, 1>{});
      else mv_tiles(std::integral_constant<int, 2>{});
      // the stores sit on the common path, so every path issues the same
      // count after the prefetch and the stage's waits stay loose.  A 4x4
      // transpose inside each quad of lanes (two DPP butterfly stages) turns
      // lane (token 4 lq + q, column lr) into (token 4 lq + lane % 4,
      // columns 4 (lr / 4) .. +4), one vector store per row tile
      const bool x1 = lane & 1, x2 = lane & 2;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 qs = QSl[(it * 4 + rr) * 64 + lane];
        float o[4] = {es[0] * qs.x + mv[rr][0], es[1] * qs.y + mv[rr][1], es[2] * qs.z + mv[rr][2],
                      es[3] * qs.w + mv[rr][3]};
#pragma unroll
        for (int p = 0; p < 4; p += 2) {  // slot bit 0 <-> lane bit 0
          const float w = dpp<DPP_XOR1>(x1 ? o[p] : o[p + 1]);
          if (x1) o[p] = w;
          else o[p + 1] = w;
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {  // slot bit 1 <-> lane bit 1
          const float w = dpp<DPP_XOR2>(x2 ? o[p] : o[p + 2]);
          if (x2) o[p] = w;
          else o[p + 2] = w;
        }
        const size_t oi = (tok0 + it * 16 + 4 * lq + (lane & 3)) * HV + size_t(h) * a.DV + r0 + rr * 16 + 4 * (lr >> 2);
        if constexpr (OUT_BF16)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + oi) =
              make_uint2(f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                         f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16));
        else
          *reinterpret_cast<float4*>(static_cast<float*>(a.o) + oi) = make_float4(o[0], o[1], o[2], o[3]);
      }
      // stage chunk c + 1, prefetch c + 2; the prefetch is issued on every
      // path (the tail re-reads the last chunk) so the stage's waits count
      // past the output stores on entry and in the loop alike
      if (c + 1 < NC) stage(par ^ 1);
      load(c + 2 < NC ? c + 2 : NC - 1);
      __syncthreads();
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
