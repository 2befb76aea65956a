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
//   state   -- one workgroup per (sequence, head, 64 rows of d_v), one
//              barrier per chunk.  Four state waves hold 16 rows each of the
//              fp32 state as MFMA accumulators (eight 16x16 tiles of S^T),
//              form Q S0^T from them and update them in place; four helper
//              waves build the decay matrix and M V, and write a chunk's
//              output one chunk later.  All products on bf16 MFMA: codes and
//              V are exact in bf16; the state, the decayed scaled V and the
//              decay matrix enter as two bf16 parts each (16 significant
//              bits, errors near 1e-5 relative).
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
// D / 32 lanes per row of D = 128 or 64 elements (32 elements each): five
// butterfly stages inside the lane, the last one or two across the lanes
// through DPP.  Output rows are 128 wide; a 64-element row is widened with
// zeros (the state kernel's operands; the zeros change no product).
constexpr int OP_THREADS = 256;
constexpr int OP_E = 32;

struct OperandArgs {
  const uint16_t* x[2];  // q, k rows [rows][128] bf16
  int8_t* codes[2];      // [rows][128]
  float* scales[2];      // [rows]
  uint16_t* rot[2];      // non-null: write the rotated rows as bf16 [rows][128] instead of codes
  int64_t rows;
  bool wht;
};

template <int D>
__global__ __launch_bounds__(OP_THREADS) void ssd_operand_kernel(OperandArgs a) {
  constexpr int OP_LPR = D / OP_E;
  const int op = blockIdx.y;
  const int tid = threadIdx.x;
  const int li = tid % OP_LPR;
  const int64_t row = int64_t(blockIdx.x) * (OP_THREADS / OP_LPR) + tid / OP_LPR;
  const bool valid = row < a.rows;
  float v[OP_E];
  const uint4* src = reinterpret_cast<const uint4*>(a.x[op] + row * D + li * OP_E);
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
    if constexpr (OP_LPR == 4) {
#pragma unroll
      for (int i = 0; i < OP_E; ++i) {
        const float o = dpp<DPP_XOR2>(v[i]);
        v[i] = up2 ? (o - v[i]) : (v[i] + o);
      }
    }
    constexpr float inv_sqrt = D == 128 ? 0.08838834764831845f : 0.125f;  // 1/sqrt(D)
#pragma unroll
    for (int i = 0; i < OP_E; ++i) v[i] *= inv_sqrt;
  }
  if (a.rot[op]) {  // bf16 operands (rotated or not; nearest even), no quantization
    if (!valid) return;
    uint4* dst = reinterpret_cast<uint4*>(a.rot[op] + row * SDK + li * OP_E);
#pragma unroll
    for (int p = 0; p < OP_E / 8; ++p) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = f32_to_bf16_bits(v[8 * p + 2 * i]) | (f32_to_bf16_bits(v[8 * p + 2 * i + 1]) << 16);
      dst[p] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if constexpr (D == 64) {  // the zero half of the row
      uint4* dz = reinterpret_cast<uint4*>(a.rot[op] + row * SDK + 64 + li * OP_E);
#pragma unroll
      for (int p = 0; p < OP_E / 8; ++p) dz[p] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
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
  if constexpr (D == 64) {  // the zero half of the row
    uint4* dz = reinterpret_cast<uint4*>(a.codes[op] + row * SDK + 64 + li * OP_E);
#pragma unroll
    for (int p = 0; p < OP_E / 16; ++p) dz[p] = make_uint4(0u, 0u, 0u, 0u);
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
constexpr int JP = 72;    // bf16 pitch of the V^T rows

// LDS carve (bytes); [2] = by chunk parity
constexpr int OFF_Q = 0;                          // q codes [2][64][QP] bf16
constexpr int OFF_K = OFF_Q + 2 * SC * QP * 2;    // k codes [2][64][QP] bf16
constexpr int OFF_KT = OFF_K + 2 * SC * QP * 2;   // k codes transposed [2][128][64], xor-swizzled granules
constexpr int OFF_V = OFF_KT + 2 * SDK * SC * 2;  // V^T [2][64 rows][JP] bf16
constexpr int OFF_QS = OFF_V + 2 * SRW * JP * 2;  // Q S0^T tiles [2][4 row tiles][4 token tiles][64 lanes] float4
constexpr int OFF_F = OFF_QS + 2 * SC * SRW * 4;  // g, exp(g), exp(g_C - g), sq, sk [2][5][64]
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

__device__ __forceinline__ bf16x4 lds4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

__device__ __forceinline__ bf16x8 cat8(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 int8 codes (two words) -> 8 bf16 packed in four words
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4v i8x8_bf16_u4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(u32x4v, i8x8_to_bf16(make_uint2(lo, hi)));
}

// Per workgroup (sequence, head, 64 rows of d_v), eight waves; wave w runs on
// SIMD w % 4, so each state wave shares its SIMD with one helper wave.
//   state waves 0..3 -- rows 16 w .. +16 of the state, all 128 columns, as
//     fp32 accumulators S^T[d][r] (eight 16x16 tiles).  A 32-wide k step
//     takes its eight k slots from two output tiles (slots 4h + q of lane
//     group g <-> index (2 ks + h) 16 + 4 g + q), so the state tiles feed
//     Q S0^T as B operands straight from registers, and so do the lanes' own
//     W = (V o d o sk)^T values in the update; A operands (Q, K^T) are read
//     from LDS as two 8-byte halves.  Per chunk: Q S0^T (published for the
//     helpers), S^T = e_C S^T + K^T W.  Nothing here waits on another wave.
//     They also stage the next chunk's k codes (as bf16), K^T and V^T and
//     load the one after.
//   helper waves 4..7 -- token tile it = w - 4: M = L o (sq sk Q K^T) for the
//     tiles (it, <= it) and M V for all rows (in registers), and a chunk
//     later the output e sq Q S0^T + M V; they also stage the next chunk's q
//     codes and per-token scalars and load the one after.
// The state's products take S and W as two bf16 parts each (16 significant
// bits), M likewise; the codes and V are exact in bf16.  One barrier per chunk.
template <bool I8, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void ssd_state_kernel(SsdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __bf16* const Qb = reinterpret_cast<__bf16*>(lds + OFF_Q);
  __bf16* const Kb = reinterpret_cast<__bf16*>(lds + OFF_K);
  __bf16* const KTb = reinterpret_cast<__bf16*>(lds + OFF_KT);
  __bf16* const Vtb = reinterpret_cast<__bf16*>(lds + OFF_V);
  float4* const QSl = reinterpret_cast<float4*>(lds + OFF_QS);
  float* const Fb = reinterpret_cast<float*>(lds + OFF_F);

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

  // prefetch mapping (256 lanes per role, u = tid % 256): k as token pair jp,
  // 16 dims 16 g8 ..; v as token pair jp, rows 8 g8 ..; q as token u / 4, 32
  // dims; the scalars of token u % 64.  The state waves load and stage k, K^T
  // and V^T, the helper waves q and the per-token scalars.
  const int u = tid & 255;
  const int jp = u & 31, g8 = u >> 5;
  const int qt = u >> 2, qd = (u & 3) * 32;
  // (clang vector types: arrays of HIP's uint4 are copied through memory)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

  if (wave < 4) {
    // ================================================================ state waves
    const int rt = wave;
    f32x4 S[8];  // S^T tiles: column r = 16 rt + lr, rows d = 16 dt + 4 lq + q
#pragma unroll
    for (int d = 0; d < 8; ++d) S[d] = {0.f, 0.f, 0.f, 0.f};
    u32x4 ka[2], kb[2], va, vb;
    auto load_kv = [&](int c) __attribute__((always_inline)) {
      const size_t t0 = tokb + size_t(c) * SC;
      const size_t ko = (t0 + 2 * jp) * HK + size_t(h) * SDK + 16 * g8;
      if constexpr (I8) {
        const int8_t* kp = static_cast<const int8_t*>(a.k) + ko;
        ka[0] = *reinterpret_cast<const u32x4*>(kp);
        kb[0] = *reinterpret_cast<const u32x4*>(kp + HK);
      } else {
        const uint16_t* kp = static_cast<const uint16_t*>(a.k) + ko;
        ka[0] = *reinterpret_cast<const u32x4*>(kp);
        ka[1] = *reinterpret_cast<const u32x4*>(kp + 8);
        kb[0] = *reinterpret_cast<const u32x4*>(kp + HK);
        kb[1] = *reinterpret_cast<const u32x4*>(kp + HK + 8);
      }
      const uint16_t* vp = a.v + (t0 + 2 * jp) * HV + size_t(h) * a.DV + r0 + 8 * g8;
      va = *reinterpret_cast<const u32x4*>(vp);
      vb = *reinterpret_cast<const u32x4*>(vp + HV);
    };
    auto stage_kv = [&](int par) __attribute__((always_inline)) {
      __bf16* Kc = Kb + par * SC * QP;
      u32x4 k0[2], k1[2];
      if constexpr (I8) {
        k0[0] = i8x8_bf16_u4(ka[0][0], ka[0][1]);
        k0[1] = i8x8_bf16_u4(ka[0][2], ka[0][3]);
        k1[0] = i8x8_bf16_u4(kb[0][0], kb[0][1]);
        k1[1] = i8x8_bf16_u4(kb[0][2], kb[0][3]);
      } else {
        k0[0] = ka[0];
        k0[1] = ka[1];
        k1[0] = kb[0];
        k1[1] = kb[1];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        *reinterpret_cast<u32x4*>(Kc + (2 * jp) * QP + 16 * g8 + 8 * e) = k0[e];
        *reinterpret_cast<u32x4*>(Kc + (2 * jp + 1) * QP + 16 * g8 + 8 * e) = k1[e];
      }
      {  // k^T: dword = tokens (2 jp, 2 jp + 1) of dim 16 g8 + e
        uint32_t* kt = reinterpret_cast<uint32_t*>(KTb + par * SDK * SC);
        const uint32_t w0[8] = {k0[0][0], k0[0][1], k0[0][2], k0[0][3], k0[1][0], k0[1][1], k0[1][2], k0[1][3]};
        const uint32_t w1[8] = {k1[0][0], k1[0][1], k1[0][2], k1[0][3], k1[1][0], k1[1][1], k1[1][2], k1[1][3]};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          kt[kt_at(16 * g8 + e, 2 * jp) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
        }
      }
      {  // V^T: rows 8 g8 + e, tokens (2 jp, 2 jp + 1)
        uint32_t* vt = reinterpret_cast<uint32_t*>(Vtb + par * SRW * JP);
        const uint32_t w0[4] = {va[0], va[1], va[2], va[3]}, w1[4] = {vb[0], vb[1], vb[2], vb[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          vt[((8 * g8 + e) * JP + 2 * jp) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
        }
      }
    };
    if (NC > 0) {
      load_kv(0);
      stage_kv(0);
      load_kv(NC > 1 ? 1 : 0);
    }
    __syncthreads();  // chunk 0 staged
    for (int c = 0; c < NC; ++c) {
      const int par = c & 1;
      const __bf16* Qc = Qb + par * SC * QP;
      const __bf16* KT = KTb + par * SDK * SC;
      const __bf16* Vt = Vtb + par * SRW * JP;
      const float* F = Fb + par * 5 * SC;
      // A operands are read ahead of their products, which then issue back
      // to back: Q rows of the four token tiles here, K^T rows below
      bf16x8 qa[4][4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const __bf16* qr = Qc + (ti * 16 + lr) * QP + ks * 32 + 4 * lq;
          qa[ti][ks] = cat8(lds4(qr), lds4(qr + 16));
        }
      // W = V o d o sk for this row tile, tokens (2 ks + hh) 16 + 4 lq + q
      bf16x8 wp[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float x[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int j0 = (2 * ks + hh) * 16 + 4 * lq;
          const uint2 vw = *reinterpret_cast<const uint2*>(Vt + (rt * 16 + lr) * JP + j0);
          const float4 d4 = *reinterpret_cast<const float4*>(F + 2 * SC + j0);
          const float4 k4 = *reinterpret_cast<const float4*>(F + 4 * SC + j0);
          x[4 * hh + 0] = bf16_lo(vw.x) * (d4.x * k4.x);
          x[4 * hh + 1] = bf16_hi(vw.x) * (d4.y * k4.y);
          x[4 * hh + 2] = bf16_lo(vw.y) * (d4.z * k4.z);
          x[4 * hh + 3] = bf16_hi(vw.y) * (d4.w * k4.w);
        }
        split2t(x, wp[0][ks], wp[1][ks]);
      }
      // S0 as B operands (two parts)
      bf16x8 sp[2][4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float x[8] = {S[2 * ks][0], S[2 * ks][1], S[2 * ks][2], S[2 * ks][3],
                            S[2 * ks + 1][0], S[2 * ks + 1][1], S[2 * ks + 1][2], S[2 * ks + 1][3]};
        split2t(x, sp[0][ks], sp[1][ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- Q S0^T for the four token tiles (published for the helpers)
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          acc = mfma16(qa[ti][ks], sp[1][ks], acc);
          acc = mfma16(qa[ti][ks], sp[0][ks], acc);
        }
        QSl[((par * 4 + rt) * 4 + ti) * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
      bf16x8 ka[8][2];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int d = dt * 16 + lr, j = ks * 32 + 4 * lq;
          ka[dt][ks] = cat8(lds4(KT + kt_at(d, j)), lds4(KT + kt_at(d, j + 16)));
        }
      __builtin_amdgcn_sched_barrier(0);
      // ---- S^T = e_C S^T + K^T W
      const float eC = F[SC + SC - 1];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        f32x4 acc = S[dt];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] *= eC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          acc = mfma16(ka[dt][ks], wp[1][ks], acc);
          acc = mfma16(ka[dt][ks], wp[0][ks], acc);
        }
        S[dt] = acc;
      }
      // stage k, K^T, V^T of chunk c + 1 into the other buffer, load c + 2
      // (unconditionally, the index clamped: every path issues the same loads)
      if (c + 1 < NC) stage_kv(par ^ 1);
      load_kv(c + 2 < NC ? c + 2 : NC - 1);
      __syncthreads();
    }
    // final state rows r0 + 16 rt + lr, columns d: S^T tile layout
    float* dst = a.state + ((size_t(b) * a.H + h) * a.DV + r0 + rt * 16 + lr) * SDK;
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<float4*>(dst + d * 16 + 4 * lq) = make_float4(S[d][0], S[d][1], S[d][2], S[d][3]);
    return;
  }

  // ================================================================ helper waves
  const int it = wave - 4;  // token tile
  u32x4 qw[4];
  float av = 1.f, sqv = 1.f, skv = 1.f;
  auto load = [&](int c) __attribute__((always_inline)) {
    const size_t t0 = tokb + size_t(c) * SC;
    const size_t qo = (t0 + qt) * HK + size_t(h) * SDK + qd;
    if constexpr (I8) {
      const int8_t* qp = static_cast<const int8_t*>(a.q) + qo;
      qw[0] = *reinterpret_cast<const u32x4*>(qp);
      qw[1] = *reinterpret_cast<const u32x4*>(qp + 16);
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qo;
#pragma unroll
      for (int e = 0; e < 4; ++e) qw[e] = *reinterpret_cast<const u32x4*>(qp + 8 * e);
    }
    {  // every helper lane loads, so each load is issued on every path
      const size_t t = (t0 + (u & 63)) * a.H + h;
      av = a.alpha[t];
      if constexpr (I8) {
        sqv = a.sq[t];
        skv = a.sk[t];
      }
    }
  };
  auto stage = [&](int par) __attribute__((always_inline)) {
    __bf16* Qc = Qb + par * SC * QP;
    u32x4 q8[4];
    if constexpr (I8) {
      q8[0] = i8x8_bf16_u4(qw[0][0], qw[0][1]);
      q8[1] = i8x8_bf16_u4(qw[0][2], qw[0][3]);
      q8[2] = i8x8_bf16_u4(qw[1][0], qw[1][1]);
      q8[3] = i8x8_bf16_u4(qw[1][2], qw[1][3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) q8[e] = qw[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(Qc + qt * QP + qd + 8 * e) = q8[e];
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

  if (NC > 0) {
    load(0);
    stage(0);
    load(NC > 1 ? 1 : 0);
  }
  __syncthreads();
  bf16x8 mA[2][2];  // M (tiles (it, 2 ks), (it, 2 ks + 1)) as A operands, hi and lo parts
  f32x4 mv[4];      // M V for the four row tiles
  float es[4];      // e_i sq_i of this wave's tokens
  auto output = [&](int c) {  // O of chunk c = e sq Q S0^T + M V
    const int par = c & 1;
    const size_t tok0 = tokb + size_t(c) * SC;
    const bool x1 = lane & 1, x2 = lane & 2;
    float4 qsv[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) qsv[rr] = QSl[((par * 4 + rr) * 4 + it) * 64 + lane];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 qs = qsv[rr];
      float o[4] = {es[0] * qs.x + mv[rr][0], es[1] * qs.y + mv[rr][1], es[2] * qs.z + mv[rr][2],
                    es[3] * qs.w + mv[rr][3]};
      // a 4x4 transpose inside each quad of lanes (two DPP butterfly stages)
      // turns lane (token 4 lq + q, row lr) into (token 4 lq + lane % 4,
      // rows 4 (lr / 4) .. +4), one vector store per row tile
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
  };
  for (int c = 0; c < NC; ++c) {
    const int par = c & 1;
    const __bf16* Qc = Qb + par * SC * QP;
    const __bf16* Kc = Kb + par * SC * QP;
    const __bf16* Vt = Vtb + par * SRW * JP;
    const float* F = Fb + par * 5 * SC;
    if (c > 0) output(c - 1);
    // ---- M = L o (sq sk Q K^T) for tiles (it, jt <= it): the tile
    //      D[j][i] = ck_j . cq_i holds tokens j = jt 16 + 4 lq + q of query i
    {
      const int i = it * 16 + lr;
      const float gi = F[i], si = F[3 * SC + i];
      // operands up front: the query row once, the key rows of all four
      // tiles (every helper takes the same branch-free path; tiles above the
      // diagonal come out zero through the mask, and the busiest helper,
      // it = 3, needs all four anyway)
      bf16x8 qo[4], ko[4][4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qo[ks] = lds_bf16x8(Qc + i * QP + ks * 32 + 8 * lq);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ko[jt][ks] = lds_bf16x8(Kc + (jt * 16 + lr) * QP + ks * 32 + 8 * lq);
      float m[4][4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16(ko[jt][ks], qo[ks], acc);
        const float4 g4 = *reinterpret_cast<const float4*>(F + jt * 16 + 4 * lq);
        const float4 k4 = *reinterpret_cast<const float4*>(F + 4 * SC + jt * 16 + 4 * lq);
        const float gj[4] = {g4.x, g4.y, g4.z, g4.w}, sj[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = jt * 16 + 4 * lq + q;
          m[jt][q] = (j <= i) ? exp_dec(gi - gj[q]) * (si * sj[q]) * acc[q] : 0.f;
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float mm[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) mm[e] = m[2 * ks + (e >> 2)][e & 3];
        split2t(mm, mA[ks][0], mA[ks][1]);
      }
    }
    // ---- M V for the four row tiles; e sq of this wave's tokens
    bf16x8 vo[4][2];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* vr = Vt + (rr * 16 + lr) * JP + ks * 32 + 4 * lq;
        vo[rr][ks] = cat8(lds4(vr), lds4(vr + 16));
      }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {  // steps past the diagonal multiply zeros of M
        acc = mfma16(mA[ks][1], vo[rr][ks], acc);
        acc = mfma16(mA[ks][0], vo[rr][ks], acc);
      }
      mv[rr] = acc;
    }
    {
      const int i0 = it * 16 + 4 * lq;
      const float4 e4 = *reinterpret_cast<const float4*>(F + SC + i0);
      const float4 q4 = *reinterpret_cast<const float4*>(F + 3 * SC + i0);
      es[0] = e4.x * q4.x;
      es[1] = e4.y * q4.y;
      es[2] = e4.z * q4.z;
      es[3] = e4.w * q4.w;
    }
    // stage chunk c + 1, prefetch c + 2; the prefetch is issued on every
    // path (the tail re-reads the last chunk) so the stage's waits count
    // past the output stores alike
    if (c + 1 < NC) stage(par ^ 1);
    load(c + 2 < NC ? c + 2 : NC - 1);
    __syncthreads();
  }
  if (NC > 0) output(NC - 1);
}

size_t ssd_rows(const PrefillLaunch& L) { return size_t(L.B) * L.T * L.H; }

// operand rows (int8 codes and scales, or bf16 rotated / widened rows), then
// at d_k = 64 the state of 128 columns whose first 64 are copied out
size_t ssd_operand_bytes(const PrefillLaunch& L) {
  const size_t rows = ssd_rows(L);
  if (L.int8_qk) return 2 * rows * SDK + 2 * rows * 4;  // q codes, k codes, q scales, k scales
  if (L.wht || L.d_k == 64) return 2 * rows * SDK * 2;  // rotated and/or widened q, k (bf16)
  return 0;
}
size_t ssd_state_pad_bytes(const PrefillLaunch& L) {
  return L.d_k == 64 ? size_t(L.B) * L.H * L.d_v * SDK * 4 : 0;
}

// [bh][d_v][128] -> [bh][d_v][64]: the first 64 columns of each state row
__global__ __launch_bounds__(256) void ssd_state_unpad_kernel(const float* ps, float* s, int64_t rows) {
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < rows * 16; e += int64_t(gridDim.x) * 256)
    reinterpret_cast<float4*>(s + (e / 16) * 64)[e % 16] = reinterpret_cast<const float4*>(ps + (e / 16) * SDK)[e % 16];
}

template <int D>
hipError_t launch_operands(const OperandArgs& oa, size_t rows, hipStream_t stream) {
  constexpr int rpb = OP_THREADS / (D / OP_E);  // rows per workgroup
  hipLaunchKernelGGL(ssd_operand_kernel<D>, dim3(unsigned((rows + rpb - 1) / rpb), 2), dim3(OP_THREADS), 0, stream, oa);
  return hipGetLastError();
}

}  // namespace

size_t prefill_ssd_workspace_bytes(const PrefillLaunch& L) {
  return (ssd_operand_bytes(L) + 255) / 256 * 256 + ssd_state_pad_bytes(L);
}

hipError_t launch_prefill_ssd(const PrefillLaunch& L, hipStream_t stream) {
  const size_t rows = ssd_rows(L);
  const void* qsrc = L.q;
  const void* ksrc = L.k;
  const float* sq = nullptr;
  const float* sk = nullptr;
  auto operands = [&](const OperandArgs& oa) {
    return L.d_k == 64 ? launch_operands<64>(oa, rows, stream) : launch_operands<128>(oa, rows, stream);
  };
  if (L.int8_qk && rows > 0) {
    int8_t* cq = static_cast<int8_t*>(L.workspace);
    int8_t* ck = cq + rows * SDK;
    float* fq = reinterpret_cast<float*>(ck + rows * SDK);
    float* fk = fq + rows;
    OperandArgs oa{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k)}, {cq, ck}, {fq, fk},
                   {nullptr, nullptr}, int64_t(rows), L.wht};
    if (hipError_t e = operands(oa)) return e;
    qsrc = cq;
    ksrc = ck;
    sq = fq;
    sk = fk;
  } else if ((L.wht || L.d_k == 64) && rows > 0) {  // rotated and/or widened bf16 operands
    uint16_t* rq = static_cast<uint16_t*>(L.workspace);
    uint16_t* rk = rq + rows * SDK;
    OperandArgs oa{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k)}, {nullptr, nullptr},
                   {nullptr, nullptr}, {rq, rk}, int64_t(rows), L.wht};
    if (hipError_t e = operands(oa)) return e;
    qsrc = rq;
    ksrc = rk;
  }
  float* state = L.state_f32;
  if (L.d_k == 64)
    state = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + (ssd_operand_bytes(L) + 255) / 256 * 256);
  SsdArgs s{qsrc, ksrc, sq, sk, static_cast<const uint16_t*>(L.v), L.alpha, L.o, state,
            L.B, L.T, L.H, L.d_v};
  const unsigned grid = unsigned(L.B) * L.H * (L.d_v / SRW);
  void (*kern)(SsdArgs) = L.int8_qk ? (L.out_bf16 ? &ssd_state_kernel<true, true> : &ssd_state_kernel<true, false>)
                                    : (L.out_bf16 ? &ssd_state_kernel<false, true> : &ssd_state_kernel<false, false>);
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, SSD_LDS))
    return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), SSD_LDS, stream, s);
  if (hipError_t e = hipGetLastError()) return e;
  if (L.d_k == 64) {
    const int64_t srows = int64_t(L.B) * L.H * L.d_v;
    hipLaunchKernelGGL(ssd_state_unpad_kernel, dim3(unsigned(srows * 16 / 256 + 1 < 4096 ? srows * 16 / 256 + 1 : 4096)),
                       dim3(256), 0, stream, state, L.state_f32, srows);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdnq
