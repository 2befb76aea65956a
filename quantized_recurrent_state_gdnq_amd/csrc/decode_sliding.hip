// Decode step of the Pure-Write sliding window on gfx950 ("Low-Bit GDN
// Recurrent-State Quantization: Global Gradient-aware Allocation and
// Pure-Write Sliding Windows", abstract: recent pure writes are kept apart,
// propagated through the full GDN transition, and merged into the low-bit
// historical state only once they leave the window).
//
// State per head: the historical part H (int8 codes + row scales) and a ring
// of the last W raw writes (k, v, alpha, beta).  Write i contributes
// beta_i v_i k~_i^T with k~_i = A_t ... A_{i+1} k_i, A_j = alpha_j (I -
// beta_j k_j k_j^T).  Per token t:
//   H' = deq(H) A_t (+ beta_l v_l k~_l^T for the write l that leaves a full
//   window), o_t = (H' + window) q_t, H = quantize(H') every token; the token's
//   write takes the ring slot of the write that left.
// With A symmetric the output unrolls as in the tumbling decode:
//   o = deq(H) (A_t q) + sum_j c_j v_j,  y = q; for j = t, newest, ..., oldest:
//   c_j = beta_j (k_j . y),  y <- alpha_j (y - c_j k_j)
// (the historical part takes only the current transition), and the leaving
// key is propagated forward through the later writes and the current one.
//
// One workgroup per head.  Phase 1: the window's keys and values go to LDS
// (oldest first), wave 0 loads q and k (rotated under WHT).  Phase 2: wave 0
// runs the backward sweep, wave 1 propagates the leaving key.  Phase 3: every
// row takes the transition, absorbs the leaving write, is requantized, and
// gives its output.
#include <hip/hip_runtime.h>

#include "decode_impl.h"

namespace gdnq {

namespace {

constexpr int SL_THREADS = 256;

// N = 1 or 2 consecutive inputs (bf16 or fp32) starting at element i
template <bool BF16, int N>
__device__ __forceinline__ void load_in_vec_n(const void* p, size_t i, float (&x)[N]) {
  if constexpr (BF16 && N == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
    x[0] = bf16_lo(w);
    x[1] = bf16_hi(w);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] = load_in<BF16>(p, i + e);
  }
}
constexpr int SL_WMAX = 64;

struct SlidingArgs {
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

// Three workgroups per CU: the window's keys and values take W (d_k + d_v)
// fp32 of LDS, sized by the call's window (8 KB at W = 8, d = 128), and the
// registers are held to three waves per SIMD (at four, phase 3's 64 columns
// per thread spill), so a CU overlaps the phases of three heads.
template <int DK, int DV, bool IN_BF16, bool OUT_BF16, bool WHT>
__global__ __launch_bounds__(SL_THREADS, 3) void sliding_kernel(SlidingArgs a) {
  constexpr int EK = DK / 64;          // key elements per lane (waves 0, 1)
  constexpr int TPR = SL_THREADS / DV; // threads per state row (phase 3)
  constexpr int CPT = DK / TPR;        // columns per thread
  static_assert(CPT % 16 == 0, "codes load in 16-byte words");
  extern __shared__ float sl_dyn[];
  float* const Kw = sl_dyn;                // window keys [W][DK], oldest first
  float* const Vw = sl_dyn + a.W * DK;     // window values [W][DV], oldest first
  __shared__ float aw[SL_WMAX], bw[SL_WMAX], cw[SL_WMAX + 1];
  __shared__ float qs[DK], ks[DK], y1[DK], kl[DK];
  __shared__ float cur[4];  // alpha_t, beta_t, c_t, leaving beta

  const int W = a.W;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int f = a.fill_in[b];
  f = f < 0 ? 0 : (f > 2 * W - 1 ? 2 * W - 1 : f);  // out of range is a data error; stay in bounds
  const bool full = f >= W;
  const int n = full ? W : f;       // writes in the window before this token
  const int p = full ? f - W : f;   // ring slot of the oldest write (full), or of the next write
  const size_t ring = size_t(bh) * W;

  // ---- phase 1: the window, oldest first (write i in ring slot (p + i) % W when full)
  for (int e = tid; e < n * (DK / 4); e += SL_THREADS) {
    const int i = e / (DK / 4), c = 4 * (e % (DK / 4));
    const int s = full ? (p + i) % W : i;
    *reinterpret_cast<float4*>(Kw + i * DK + c) = *reinterpret_cast<const float4*>(a.buf_k + (ring + s) * DK + c);
  }
  for (int e = tid; e < n * (DV / 4); e += SL_THREADS) {
    const int i = e / (DV / 4), c = 4 * (e % (DV / 4));
    const int s = full ? (p + i) % W : i;
    *reinterpret_cast<float4*>(Vw + i * DV + c) = *reinterpret_cast<const float4*>(a.buf_v + (ring + s) * DV + c);
  }
  if (tid < n) {
    const int s = full ? (p + tid) % W : tid;
    aw[tid] = a.buf_alpha[ring + s];
    bw[tid] = a.buf_beta[ring + s];
  }
  if (wave == 0) {
    float qv[EK], kv[EK];
    load_in_vec_n<IN_BF16, EK>(a.q, size_t(bh) * DK + lane * EK, qv);
    load_in_vec_n<IN_BF16, EK>(a.k, size_t(bh) * DK + lane * EK, kv);
    if constexpr (WHT) {
      fwht_group<EK, 64>(qv, lane);
      fwht_group<EK, 64>(kv, lane);
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      qs[lane * EK + e] = qv[e];
      ks[lane * EK + e] = kv[e];
    }
    if (lane == 0) {
      cur[0] = a.alpha[bh];
      cur[1] = a.beta[bh];
    }
  }
  __syncthreads();
  const float alpha_t = cur[0], beta_t = cur[1];

  // ---- phase 2: wave 0 the backward sweep, wave 1 the leaving key
  if (wave == 0) {
    float y[EK], kt[EK];
    float p0 = 0.f;
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      y[e] = qs[lane * EK + e];
      kt[e] = ks[lane * EK + e];
      p0 += kt[e] * y[e];
    }
    const float c_t = beta_t * wave_allreduce_sum(p0);
#pragma unroll
    for (int e = 0; e < EK; ++e) y[e] = alpha_t * (y[e] - c_t * kt[e]);
#pragma unroll
    for (int e = 0; e < EK; ++e) y1[lane * EK + e] = y[e];  // A_t q: the historical part's vector
    if (lane == 0) cur[2] = c_t;
    float creg = 0.f;  // lane i: c of window write i
    for (int i = n - 1; i >= 0; --i) {
      float pk = 0.f, kk[EK];
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        kk[e] = Kw[i * DK + lane * EK + e];
        pk += kk[e] * y[e];
      }
      const float ci = bw[i] * wave_allreduce_sum(pk);
      creg = lane == i ? ci : creg;
      const float ai = aw[i];
#pragma unroll
      for (int e = 0; e < EK; ++e) y[e] = ai * (y[e] - ci * kk[e]);
    }
    cw[lane] = creg;
  } else if (wave == 1 && !full) {
#pragma unroll
    for (int e = 0; e < EK; ++e) kl[lane * EK + e] = 0.f;  // no write leaves
    if (lane == 0) cur[3] = 0.f;
  } else if (wave == 1) {
    // the oldest write leaves: its key through the later writes, oldest
    // first, then through the current token's transition
    float x[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e) x[e] = Kw[lane * EK + e];
    for (int j = 1; j <= n; ++j) {
      float kk[EK], aj, bj;
      if (j < n) {
#pragma unroll
        for (int e = 0; e < EK; ++e) kk[e] = Kw[j * DK + lane * EK + e];
        aj = aw[j];
        bj = bw[j];
      } else {
#pragma unroll
        for (int e = 0; e < EK; ++e) kk[e] = ks[lane * EK + e];
        aj = alpha_t;
        bj = beta_t;
      }
      float pk = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) pk += kk[e] * x[e];
      const float d = wave_allreduce_sum(pk);
#pragma unroll
      for (int e = 0; e < EK; ++e) x[e] = aj * (x[e] - bj * d * kk[e]);
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) kl[lane * EK + e] = x[e];
    if (lane == 0) cur[3] = bw[0];
  }
  __syncthreads();

  // ---- phase 3: rows.  Thread -> row tid / TPR, columns (tid % TPR) * CPT ..
  const int r = tid / TPR, seg = tid % TPR;
  const size_t row = size_t(bh) * DV + r;
  const float c_t = cur[2];
  const float vl = full ? Vw[r] : 0.f;  // the leaving write's value (window write 0)
  const float lw = cur[3] * vl;         // its beta times its value (0 when none leaves)
  const float s_old = a.scales[row];
  float hv[CPT];
  {
    const int8_t* src = a.codes + row * DK + seg * CPT;
#pragma unroll
    for (int w4 = 0; w4 < CPT / 16; ++w4) {
      const uint4 u = *reinterpret_cast<const uint4*>(src + 16 * w4);
      const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) hv[16 * w4 + 4 * qq + bb] = i8_at(ww[qq], bb);
    }
  }
  // output: deq(H) . (A_t q) + sum_j c_j v_j[r] + c_t v_t[r]; both products
  // on the codes, the row scale applied once to each sum
  float po = 0.f, hk = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    po = fmaf(hv[c], y1[seg * CPT + c], po);
    hk = fmaf(hv[c], ks[seg * CPT + c], hk);
  }
  po *= s_old;
  for (int i = seg; i < n; i += TPR) po = fmaf(cw[i], Vw[i * DV + r], po);
  po = group_sum<TPR>(po);
  hk = group_sum<TPR>(hk);
  const float v_t = (seg == 0) ? load_in<IN_BF16>(a.v, row) : 0.f;
  // historical row through the transition, plus the leaving write; requantize:
  // alpha (s c - beta (h . k) k) + lw kl with h . k = s (c . k), the scale
  // folded into the per-row factors
  const float as = alpha_t * s_old, bk = alpha_t * beta_t * (s_old * hk);
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const float x = fmaf(as, hv[c], fmaf(-bk, ks[seg * CPT + c], lw * kl[seg * CPT + c]));
    hv[c] = x;
    amax = fmaxf(amax, fabsf(x));
  }
  amax = group_max<TPR>(amax);
  const float scale = codec_scale(amax);
  {
    // the reciprocal form of the codec (divisions only next to a rounding
    // tie): the same codes as dividing every element, at a fraction of the
    // instructions
    int8_t* dst = a.codes + row * DK + seg * CPT;
#pragma unroll
    for (int w4 = 0; w4 < CPT / 16; ++w4) {  // 16 columns at a time (one store)
      float x[16], cf[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) x[c] = hv[16 * w4 + c];
      codec_codes(x, scale, cf);
      uint4 u;
      uint32_t* uw = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        uw[qq] = pack4_i8(int(cf[4 * qq]), int(cf[4 * qq + 1]), int(cf[4 * qq + 2]), int(cf[4 * qq + 3]));
      *reinterpret_cast<uint4*>(dst + 16 * w4) = u;
    }
  }
  if (seg == 0) {
    a.scales[row] = scale;
    store_out<OUT_BF16>(a.o, row, po + c_t * v_t);
  }
  // the token's write into the ring slot (the one the leaving write held):
  // every read of that slot happened in phase 1, before the barriers
  const int slot = p;
  for (int c = tid; c < DK; c += SL_THREADS) a.buf_k[(ring + slot) * DK + c] = ks[c];
  if (tid < DV) a.buf_v[(ring + slot) * DV + tid] = load_in<IN_BF16>(a.v, size_t(bh) * DV + tid);
  if (tid == 0) {
    a.buf_alpha[ring + slot] = alpha_t;
    a.buf_beta[ring + slot] = beta_t;
    if (h == 0) a.fill_out[b] = full ? W + (p + 1) % W : f + 1;
  }
}

template <int DK, int DV, bool IB, bool OB, bool WH>
hipError_t launch_sl1(const SlidingArgs& s, hipStream_t st) {
  const dim3 grid(unsigned(s.B) * s.H), block(SL_THREADS);
  const unsigned lds = unsigned(s.W) * (DK + DV) * 4;
  const void* fn = reinterpret_cast<const void*>(&sliding_kernel<DK, DV, IB, OB, WH>);
  if (hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, SL_WMAX * (DK + DV) * 4))
    return e;
  hipLaunchKernelGGL((sliding_kernel<DK, DV, IB, OB, WH>), grid, block, lds, st, s);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_sl(const SlidingArgs& s, bool ib, bool ob, bool wht, hipStream_t st) {
#define GDNQ_SL(IB, OB, WH) return launch_sl1<DK, DV, IB, OB, WH>(s, st)
  if (ib) {
    if (ob) { if (wht) GDNQ_SL(true, true, true); else GDNQ_SL(true, true, false); }
    else { if (wht) GDNQ_SL(true, false, true); else GDNQ_SL(true, false, false); }
  } else {
    if (ob) { if (wht) GDNQ_SL(false, true, true); else GDNQ_SL(false, true, false); }
    else { if (wht) GDNQ_SL(false, false, true); else GDNQ_SL(false, false, false); }
  }
#undef GDNQ_SL
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_sliding(const DecodeLaunch& L, hipStream_t stream) {
  SlidingArgs s{L.q, L.k, L.v, L.alpha, L.beta, L.codes, L.scales,
                static_cast<float*>(L.buf_k), static_cast<float*>(L.buf_v), L.buf_alpha, L.buf_beta,
                L.fill_in, L.fill_out, L.o, L.B, L.H, L.W};
  if (L.d_k == 128 && L.d_v == 128) return launch_sl<128, 128>(s, L.in_bf16, L.out_bf16, L.wht, stream);
  if (L.d_k == 128 && L.d_v == 64) return launch_sl<128, 64>(s, L.in_bf16, L.out_bf16, L.wht, stream);
  if (L.d_k == 64 && L.d_v == 128) return launch_sl<64, 128>(s, L.in_bf16, L.out_bf16, L.wht, stream);
  return launch_sl<64, 64>(s, L.in_bf16, L.out_bf16, L.wht, stream);
}

}  // namespace gdnq
