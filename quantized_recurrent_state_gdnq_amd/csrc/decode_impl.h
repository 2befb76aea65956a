// Decode step of the per-window low-bit-state gated delta rule on gfx950
// (kernel templates; decode.hip instantiates the 8-bit state, decode_q4.hip
// the 4-bit one, so the two compile in parallel).
//
// LeapQuant (abstract): inside a window the output comes from the fixed
// low-bit state plus the window's buffered high-precision writes, and the
// state is requantized once, when the window closes.  Low-Bit GDN ...
// (abstract): the buffered writes go through the full GDN transition.
//
// Work is a list of jobs built on the device from the fills, identical in
// every workgroup of a persistent grid (workgroup g takes jobs g, g+G, ...):
//   * close jobs first: a sequence whose window closes (f + 1 == W) has each
//     head split into row blocks (rows of the state evolve independently);
//     a close job replays the W writes on its dequantized rows in fp32,
//     takes the output from that state and requantizes the rows in place;
//   * then one open job per remaining head: with A_j = alpha_j (I - beta_j
//     k_j k_j^T) (symmetric) the replay unrolls to
//         o = S_t q = S_0 y_0 + sum_j c_j v_j,
//         y = q, then for j = t, t-1, ..., 1:  c_j = beta_j (k_j . y),
//                                               y <- alpha_j (y - c_j k_j),
//     so the d_v x d_k state is read once, as int8, and never rebuilt.  One
//     wave runs that backward sweep; every wave streams int8 rows.
// Buffered keys and values are loaded into registers at the start of a job
// (bounded buffer loads: slots past the fill cost no traffic) and pass
// through LDS 16 slots at a time.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace gdnq {

constexpr int DEC_THREADS = 256;
constexpr int DEC_MAXB = 1024;   // sequences per call (fill scan results in LDS)
#ifndef DEC_CODE_LEAD
#define DEC_CODE_LEAD 1
#endif
#ifndef DEC_QUEUE
#define DEC_QUEUE 14
#endif
#ifndef DEC_WG_PER_CU
#define DEC_WG_PER_CU 3  // resident workgroups per CU (sets the register budget)
#endif
#ifndef DEC_OPEN_WAVES
#define DEC_OPEN_WAVES 1024
#endif
#ifndef DEC_QUEUE_BF16
#define DEC_QUEUE_BF16 24  // bf16 and E4M3 window buffers: half the queue registers per slot
#endif

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  int8_t* codes;
  float* scales;
  void* buf_k;  // fp32, bf16 or E4M3 codes (BUF = 0, 1, 2)
  void* buf_v;
  float* buf_alpha;
  float* buf_beta;
  const int32_t* fill_in;
  int32_t* fill_out;
  void* o;
  int B, H, W;
  int open_waves;  // waves that take open heads (the rest of the grid's waves idle)
  float* ks;       // E4M3 buffer: one scale per buffered key [B*H*W] (else unused)
  float* vs;       // and per buffered value
};

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if constexpr (BF16) return bf16_at(static_cast<const uint16_t*>(p), i);
  else return static_cast<const float*>(p)[i];
}

// N consecutive inputs starting at element i (N = 4 or 8, i a multiple of N)
template <bool BF16, int N>
__device__ __forceinline__ void load_in_vec(const void* p, size_t i, float (&x)[N]) {
  if constexpr (BF16) {
    const uint16_t* b = static_cast<const uint16_t*>(p) + i;
    if constexpr (N == 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(b);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(ww[e]);
        x[2 * e + 1] = bf16_hi(ww[e]);
      }
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(b);
      x[0] = bf16_lo(w.x);
      x[1] = bf16_hi(w.x);
      x[2] = bf16_lo(w.y);
      x[3] = bf16_hi(w.y);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
#pragma unroll
    for (int e = 0; e < N / 4; ++e) {
      const float4 v = f[e];
      x[4 * e] = v.x;
      x[4 * e + 1] = v.y;
      x[4 * e + 2] = v.z;
      x[4 * e + 3] = v.w;
    }
  }
}

// N consecutive inputs kept as raw words (RAW_WORDS<BF16, N> of them).
template <bool BF16, int N>
struct RawVec {
  static constexpr int WORDS = BF16 ? (N + 1) / 2 : N;
  uint32_t w[WORDS];
};
template <bool BF16, int N>
__device__ __forceinline__ void load_raw_vec(const void* p, size_t i, RawVec<BF16, N>& r) {
  constexpr int WORDS = RawVec<BF16, N>::WORDS;
  const char* src = static_cast<const char*>(p) + i * (BF16 ? 2 : 4);
  if constexpr (BF16 && N == 1) {  // one bf16 in the low half
    r.w[0] = *reinterpret_cast<const uint16_t*>(src);
  } else if constexpr (WORDS == 1) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(src);
  } else if constexpr (WORDS == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(src);
    r.w[0] = u.x;
    r.w[1] = u.y;
  } else {
#pragma unroll
    for (int q = 0; q < WORDS / 4; ++q) {
      const uint4 u = reinterpret_cast<const uint4*>(src)[q];
      r.w[4 * q] = u.x;
      r.w[4 * q + 1] = u.y;
      r.w[4 * q + 2] = u.z;
      r.w[4 * q + 3] = u.w;
    }
  }
}
// Converts after an empty asm that "redefines" the words: no conversion, and
// so no wait for the load, can be scheduled before this point.
template <bool BF16, int N>
__device__ __forceinline__ void unpack_raw_vec(RawVec<BF16, N>& r, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < RawVec<BF16, N>::WORDS; ++q) asm volatile("" : "+v"(r.w[q]));
#pragma unroll
  for (int q = 0; q < RawVec<BF16, N>::WORDS; ++q) {
    if constexpr (BF16 && N == 1) {
      x[0] = bf16_lo(r.w[0]);
    } else if constexpr (BF16) {
      x[2 * q] = bf16_lo(r.w[q]);
      x[2 * q + 1] = bf16_hi(r.w[q]);
    } else {
      x[q] = __uint_as_float(r.w[q]);
    }
  }
}

// Raw input bits (bf16 pattern or fp32 bits): loading without converting keeps
// the compiler from waiting on the load where it is issued.
template <bool BF16>
__device__ __forceinline__ uint32_t load_raw(const void* p, size_t i) {
  if constexpr (BF16) return static_cast<const uint16_t*>(p)[i];
  else return static_cast<const uint32_t*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ float raw_to_f32(uint32_t r) {
  asm volatile("" : "+v"(r));
  return BF16 ? __uint_as_float(r << 16) : __uint_as_float(r);
}

// Cache policy of the buffered-write and decay loads: each is read once per
// step, and as nontemporal loads the fp32 and bf16 buffers' steps ran faster
// (B=64 H=32: 27.7 -> 25.0 us with the fp32 buffer); the E4M3 buffer's
// step ran faster without.
constexpr int dec_pol(int buf) { return buf == 2 ? 0 : BUF_STREAM; }

template <bool BF16>
__device__ __forceinline__ void store_out(void* p, size_t i, float x) {
  if constexpr (BF16) __builtin_nontemporal_store(uint16_t(f32_to_bf16_bits(x)), static_cast<uint16_t*>(p) + i);
  else __builtin_nontemporal_store(x, static_cast<float*>(p) + i);
}
// rows i, i + 1 of the output in one store
typedef float f32x2v __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ void store_out2(void* p, size_t i, float x0, float x1) {
  if constexpr (BF16)
    __builtin_nontemporal_store(f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16),
                                reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + i));
  else
    __builtin_nontemporal_store(f32x2v{x0, x1}, reinterpret_cast<f32x2v*>(static_cast<float*>(p) + i));
}

// A value the compiler cannot prove wave-uniform (it comes from LDS) but is:
// moving it to a scalar register keeps all address arithmetic scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float lane_value(float x, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}

// Marks a loaded register as consumed here, so that no load of this job is
// still pending when the next job starts reusing registers (a pending load
// would make the next job wait, in order, for everything issued before it).
__device__ __forceinline__ void consume(float4 x) { asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w)); }
__device__ __forceinline__ void consume(float x) { asm volatile("" ::"v"(x)); }

// k-th set bit (0-based) of m; m must have more than k bits set.
__device__ __forceinline__ int kth_bit(uint64_t m, int k) {
  for (int i = 0; i < k; ++i) m &= m - 1;
  return __builtin_ctzll(m);
}

template <int DK, int DV>
struct DecShape {
  static constexpr int NT = DEC_THREADS;
  static constexpr int CPR = DK / 16;            // 16-code chunks per row
  static constexpr int NC = DV * CPR / NT;       // chunks per thread (open job)
  static constexpr int EK = DK / 64;             // elements of q, k per lane of a wave
  static constexpr int KF4 = DK / 4;             // float4 per key
  static constexpr int KREG = 64 * KF4 / NT;     // key float4 loads per thread
  static constexpr int VRG = DV / 4;             // float4 row groups of values
  static constexpr int VNG = NT / VRG;           // slot groups (open job)
  static constexpr int VREG = 64 / VNG;          // value float4 registers (open job)
  static constexpr int CCOL = 8;                 // state columns per thread (close job)
  static constexpr int CSEG = DK / CCOL;         // threads per state row (close job)
  static constexpr int CR = NT / CSEG;           // rows per close job
  static constexpr int RC = DV / CR;             // close jobs per head
  static constexpr int CVF4 = CR / 4;            // float4 per slot of a close job's values
  static constexpr int CVREG = (64 * CVF4 + NT - 1) / NT;
  static_assert(NC >= 1 && KREG >= 1 && VREG >= 1 && RC >= 1, "decode tiling");
  // static LDS (floats); the keys [W][DK] live in dynamic LDS
  static constexpr int XSZ = (VNG * DV > 64 * CR) ? VNG * DV : 64 * CR;
  static constexpr int L_X = 0;                   // open: partial sums [VNG][DV]; close: values [W][CR]
  static constexpr int L_Y = L_X + XSZ;           // [NT/64][DK] y per wave (open) / q (close)
  static constexpr int L_C = L_Y + (NT / 64) * DK;  // [64] c_j
  static constexpr int L_D = L_C + 64;            // [DV] row dots
  static constexpr int L_END = L_D + DV;
};

// Job list shared by every workgroup: closing sequences first (bit masks and
// prefix counts per 64 sequences), then the open heads, their sequences sorted
// by fill, longest first; plus each sequence's fill.
struct JobList {
  uint64_t* cmask;
  int* cpre;
  uint8_t* fills;
  uint16_t* order;  // open sequences, longest window first
  int B, H, RC, n_close_jobs, n_jobs;
};

struct JobId {
  int seq, h, rb, f;
};

__device__ __forceinline__ JobId job_id(const JobList& L, int job) {
  JobId j;
  if (job < L.n_close_jobs) {
    const int rank = job / (L.H * L.RC);
    j.h = (job / L.RC) % L.H;
    j.rb = job % L.RC;
    int c = 0;
    while (uniform(L.cpre[c + 1]) <= rank) ++c;
    j.seq = uniform(c * 64 + kth_bit(L.cmask[c], rank - L.cpre[c]));
  } else {
    const int oj = job - L.n_close_jobs;
    j.h = oj % L.H;
    j.rb = 0;
    j.seq = uniform(int(L.order[oj / L.H]));
  }
  j.f = uniform(L.fills[j.seq]);
  return j;
}

// The open heads of one wave, one after another.  With A_j = alpha_j (I -
// beta_j k_j k_j^T) (symmetric) the window replay unrolls to
//     o = S_0 y_0 + sum_j c_j v_j,   y = q;  for j = t, t-1, ..., 1:
//     c_j = beta_j (k_j . y),  y <- alpha_j (y - c_j k_j),
// so the int8 rows are read once and the state is never rebuilt.  The sweep
// reads each buffered key and value straight from memory through a P-deep
// register queue (bounded buffer loads: slots past the fill cost nothing)
// and accumulates c_j v_j as it goes; the int8 rows are loaded while it runs.
// The wave takes positions slot, 2NW-1-slot, 2NW+slot, ... of the open-head
// list.  (Issuing the next head's loads before a head's rows . y work was
// measured slower: the extra in-flight loads only queue behind HBM.)
template <int DK, int DV, bool IN_BF16, bool OUT_BF16, bool WHT, int BUF, int QB>
__device__ __forceinline__ void open_wave(const DecodeArgs& a, const JobList& L, int slot, int NW, int n_open,
                                          int lane, float* wy, int* pool) {
  constexpr int EK = DK / 64;    // key / query elements per lane
  constexpr int RPL = DV / 64;   // state rows per lane
  constexpr int CPU4 = 128 / QB;   // codes per 16-byte load
  constexpr int CPR = DK / CPU4;   // 16-byte loads per row
  constexpr int RB = DK * QB / 8;  // bytes per row
  constexpr int EB = BUF == 0 ? 4 : BUF == 1 ? 2 : 1;  // bytes per buffered element
  constexpr int KWD = BUF == 0 ? EK : 1;   // queue words per buffered key (per lane)
  constexpr int VWD = BUF == 0 ? RPL : 1;  // and per buffered value
  constexpr int P = BUF == 0 ? DEC_QUEUE : DEC_QUEUE_BF16;  // queue depth (sweep steps loaded ahead)
  constexpr int CODE_LEAD = DEC_CODE_LEAD;
  const int W = a.W;
  const uint32_t ko = uint32_t(lane) * EK * EB, vo = uint32_t(lane) * RPL * EB;
  // the head being swept (filled by fetch while the previous head finishes)
  JobId J;
  int bh;
  rsrc_t rk, rv;
  // raw words of a buffered key / value (fp32 bits, packed bf16 or packed
  // E4M3 codes): the queue holds these and they are widened at the step
  // that consumes them
  auto load_raw = [&](const rsrc_t& r, uint32_t o, uint32_t so, int n, uint32_t* x) __attribute__((always_inline)) {
    if (BUF == 0 && n == 2) {
      const uint2 w = bload_u2s<dec_pol(BUF)>(r, o, so);
      x[0] = w.x;
      x[1] = w.y;
    } else if (BUF == 0 || (BUF == 1 && n == 2)) {
      x[0] = __float_as_uint(bload_f1s<dec_pol(BUF)>(r, o, so));
    } else if (BUF == 1 || n == 2) {
      x[0] = bload_h1s<dec_pol(BUF)>(r, o, so);
    } else {
      x[0] = bload_b1s<dec_pol(BUF)>(r, o, so);
    }
  };
  auto load_k = [&](int j, uint32_t (&x)[KWD]) {  // j < 0 lands past the bound: reads 0, no traffic
    load_raw(rk, ko, uint32_t(j) * DK * EB, EK, x);
  };
  auto load_v = [&](int j, uint32_t (&x)[VWD]) {
    load_raw(rv, vo, uint32_t(j) * DV * EB, RPL, x);
  };
  // sc: the vector's scale (E4M3 buffer only): the widened value is
  // code * scale in fp32, exactly the value the buffer stands for
  auto widen_k = [&](const uint32_t (&x)[KWD], float (&y)[EK], float sc) __attribute__((always_inline)) {
    if constexpr (BUF == 0) {
#pragma unroll
      for (int e = 0; e < EK; ++e) y[e] = __uint_as_float(x[e]);
    } else if constexpr (BUF == 1) {
      y[0] = bf16_lo(x[0]);
      if constexpr (EK == 2) y[1] = bf16_hi(x[0]);
    } else {
      const float2 c = e4m3_unpack2(x[0], false);
      y[0] = c.x * sc;
      if constexpr (EK == 2) y[1] = c.y * sc;
    }
  };
  auto widen_v = [&](const uint32_t (&x)[VWD], float (&y)[RPL], float sc) __attribute__((always_inline)) {
    if constexpr (BUF == 0) {
#pragma unroll
      for (int e = 0; e < RPL; ++e) y[e] = __uint_as_float(x[e]);
    } else if constexpr (BUF == 1) {
      y[0] = bf16_lo(x[0]);
      if constexpr (RPL == 2) y[1] = bf16_hi(x[0]);
    } else {
      const float2 c = e4m3_unpack2(x[0], false);
      y[0] = c.x * sc;
      if constexpr (RPL == 2) y[1] = c.y * sc;
    }
  };
  uint32_t kq[P][KWD], vq[P][VWD];
  float a_slot, b_slot, alpha_t, beta_t;
  float ks_slot = 1.f, vs_slot = 1.f;  // lane j: scales of write j (E4M3 buffer)
  RawVec<IN_BF16, EK> qraw, kraw;
  RawVec<IN_BF16, RPL> vraw;
  float srow[RPL];
  // every load a head needs before its sweep: token inputs, scales and
  // per-slot decays first, then the first P buffered writes
  auto fetch = [&](int o) __attribute__((always_inline)) {
    J = job_id(L, L.n_close_jobs + o);
    bh = J.seq * a.H + J.h;
    const int fb = J.f;
    const size_t bufs = size_t(bh) * W;
    rk = make_rsrc(static_cast<const char*>(a.buf_k) + bufs * DK * EB, uint32_t(fb) * DK * EB);
    rv = make_rsrc(static_cast<const char*>(a.buf_v) + bufs * DV * EB, uint32_t(fb) * DV * EB);
    load_raw_vec<IN_BF16, EK>(a.q, size_t(bh) * DK + lane * EK, qraw);
    load_raw_vec<IN_BF16, EK>(a.k, size_t(bh) * DK + lane * EK, kraw);
    load_raw_vec<IN_BF16, RPL>(a.v, size_t(bh) * DV + lane * RPL, vraw);
#pragma unroll
    for (int i = 0; i < RPL; ++i) srow[i] = a.scales[size_t(bh) * DV + lane * RPL + i];
    alpha_t = a.alpha[bh];
    beta_t = a.beta[bh];
    a_slot = bload_f1<dec_pol(BUF)>(make_rsrc(a.buf_alpha + bufs, uint32_t(fb) * 4), uint32_t(lane) * 4);
    b_slot = bload_f1<dec_pol(BUF)>(make_rsrc(a.buf_beta + bufs, uint32_t(fb) * 4), uint32_t(lane) * 4);
    if constexpr (BUF == 2) {
      ks_slot = bload_f1<dec_pol(BUF)>(make_rsrc(a.ks + bufs, uint32_t(fb) * 4), uint32_t(lane) * 4);
      vs_slot = bload_f1<dec_pol(BUF)>(make_rsrc(a.vs + bufs, uint32_t(fb) * 4), uint32_t(lane) * 4);
    }
#pragma unroll
    for (int u = 0; u < P; ++u) {
      load_k(J.f - 1 - u, kq[u]);
      load_v(J.f - 1 - u, vq[u]);
    }
  };
  // With four waves of open heads in every workgroup, the workgroup's later
  // heads (the positions its four waves would take in rounds 1, 2, ... of
  // the deal) are a pool in LDS: a wave takes the next one, longest first,
  // when its current head's code rows are loaded, so a wave that finishes
  // early takes more of the workgroup's work.
  const int g4 = slot & ~3;  // this workgroup's first slot
  const bool pooled = (NW & 3) == 0;
  int k = 0;
  int o = slot;
  fetch(o);
  for (;;) {
    unsigned gv = 0;  // lane 0: the pool index of this wave's next head
    auto grab = [&]() { if (pooled && lane == 0) gv = unsigned(atomicAdd(pool, 1)); };
    const int f = J.f;
    const size_t v_base = size_t(bh) * DV;
    const size_t bufs_base = size_t(bh) * W;
    // the int8 rows are needed last: their loads go out when at most CODE_LEAD
    // blocks of sweep steps remain, so that early bandwidth feeds the sweeps of
    // the heads with the longest windows (they bound the step)
    uint4 cw[RPL][CPR];
    auto load_codes = [&]() {
#pragma unroll
      for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int c = 0; c < CPR; ++c)
          cw[i][c] = *reinterpret_cast<const uint4*>(a.codes + (v_base + lane * RPL + i) * RB + 16 * c);
    };

    float qv[EK], kv[EK], vcur[RPL];
    unpack_raw_vec<IN_BF16, EK>(qraw, qv);
    unpack_raw_vec<IN_BF16, EK>(kraw, kv);
    unpack_raw_vec<IN_BF16, RPL>(vraw, vcur);
    if constexpr (WHT) {
      fwht_group<EK, 64>(qv, lane);
      fwht_group<EK, 64>(kv, lane);
    }
    // the current token first, then the buffered writes newest to oldest;
    // carried as yt = y / (product of the alphas swept so far)
    float yt[EK];
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      yt[e] = qv[e];
      p += kv[e] * qv[e];
    }
    const float c_cur = beta_t * wave_allreduce_sum(p);
#pragma unroll
    for (int e = 0; e < EK; ++e) yt[e] -= c_cur * kv[e];
    float G = alpha_t;
    float acc[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) acc[i] = c_cur * vcur[i];
    // append v and k (k in the rotated basis under WHT; a bf16 buffer keeps
    // them rounded to nearest even) now, so that neither stays live through the
    // sweep: the sweep never reads slot f (its loads are bounded at f writes)
    if constexpr (BUF == 2) {
      // E4M3 vector pairs: per vector scale = absmax / 448 and codes nearest
      // to x / scale (IEEE divisions, ties to even)
      float mk = 0.f, mv = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) mk = fmaxf(mk, fabsf(kv[e]));
#pragma unroll
      for (int i = 0; i < RPL; ++i) mv = fmaxf(mv, fabsf(vcur[i]));
      const float sk = __fdiv_rn(group_max<64>(mk), 448.f);
      const float sv = __fdiv_rn(group_max<64>(mv), 448.f);
      float ck[2] = {0.f, 0.f}, cv[2] = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < EK; ++e) ck[e] = sk > 0.f ? e4m3_round(__fdiv_rn(kv[e], sk)) : 0.f;
#pragma unroll
      for (int i = 0; i < RPL; ++i) cv[i] = sv > 0.f ? e4m3_round(__fdiv_rn(vcur[i], sv)) : 0.f;
      uint8_t* bk = static_cast<uint8_t*>(a.buf_k) + (bufs_base + f) * DK + lane * EK;
      uint8_t* bv = static_cast<uint8_t*>(a.buf_v) + (bufs_base + f) * DV + lane * RPL;
      if constexpr (EK == 2) *reinterpret_cast<uint16_t*>(bk) = uint16_t(e4m3_pack2(ck[0], ck[1]));
      else bk[0] = uint8_t(e4m3_pack2(ck[0], 0.f));
      if constexpr (RPL == 2) *reinterpret_cast<uint16_t*>(bv) = uint16_t(e4m3_pack2(cv[0], cv[1]));
      else bv[0] = uint8_t(e4m3_pack2(cv[0], 0.f));
      if (lane == 0) {
        a.ks[bufs_base + f] = sk;
        a.vs[bufs_base + f] = sv;
      }
    } else if constexpr (BUF == 1) {
      uint16_t* bv = static_cast<uint16_t*>(a.buf_v) + (bufs_base + f) * DV + lane * RPL;
      uint16_t* bk = static_cast<uint16_t*>(a.buf_k) + (bufs_base + f) * DK + lane * EK;
      if constexpr (RPL == 2)
        *reinterpret_cast<uint32_t*>(bv) = f32_to_bf16_bits(vcur[0]) | (f32_to_bf16_bits(vcur[1]) << 16);
      else
        bv[0] = uint16_t(f32_to_bf16_bits(vcur[0]));
      if constexpr (EK == 2)
        *reinterpret_cast<uint32_t*>(bk) = f32_to_bf16_bits(kv[0]) | (f32_to_bf16_bits(kv[1]) << 16);
      else
        bk[0] = uint16_t(f32_to_bf16_bits(kv[0]));
    } else {
      float* bv = static_cast<float*>(a.buf_v) + (bufs_base + f) * DV + lane * RPL;
      float* bk = static_cast<float*>(a.buf_k) + (bufs_base + f) * DK + lane * EK;
#pragma unroll
      for (int i = 0; i < RPL; ++i) __builtin_nontemporal_store(vcur[i], bv + i);
#pragma unroll
      for (int e = 0; e < EK; ++e) __builtin_nontemporal_store(kv[e], bk + e);
    }
    if (lane == 0) {
      a.buf_alpha[bufs_base + f] = alpha_t;
      a.buf_beta[bufs_base + f] = beta_t;
      if (J.h == 0) a.fill_out[J.seq] = f + 1;
    }
    // one sweep step on queue slot u (write j): the slot is copied out first so
    // that its registers can take the load of write j - P at once
    auto step = [&](int u, int j, bool refill) {
      uint32_t kw[KWD], vw[VWD];
#pragma unroll
      for (int e = 0; e < KWD; ++e) asm volatile("v_mov_b32 %0, %1" : "=v"(kw[e]) : "v"(kq[u][e]));
#pragma unroll
      for (int i = 0; i < VWD; ++i) asm volatile("v_mov_b32 %0, %1" : "=v"(vw[i]) : "v"(vq[u][i]));
      float kj[EK], vj[RPL];
      widen_k(kw, kj, BUF == 2 ? lane_value(ks_slot, j) : 1.f);
      widen_v(vw, vj, BUF == 2 ? lane_value(vs_slot, j) : 1.f);
      if (refill) {
        load_k(j - P, kq[u]);
        load_v(j - P, vq[u]);
      }
      float pp = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) pp += kj[e] * yt[e];
      const float bt = lane_value(b_slot, j) * wave_allreduce_sum(pp);
#pragma unroll
      for (int e = 0; e < EK; ++e) yt[e] -= bt * kj[e];
      const float cj = bt * G;
#pragma unroll
      for (int i = 0; i < RPL; ++i) acc[i] = fmaf(cj, vj[i], acc[i]);
      G *= lane_value(a_slot, j);
    };
    // two writes at a time (slots u, u + 1 = writes j, j - 1): with
    // d_a = k_j . yt, d_b = k_{j-1} . yt and g = k_j . k_{j-1} (three
    // overlapped reductions), bt_a = beta_j d_a and
    // bt_b = beta_{j-1} (k_{j-1} . (yt - bt_a k_j)) = beta_{j-1} (d_b - bt_a g)
    auto step2 = [&](int u, int j, bool refill) {
      uint32_t kwa[KWD], kwb[KWD], vwa[VWD], vwb[VWD];
#pragma unroll
      for (int e = 0; e < KWD; ++e) {
        asm volatile("v_mov_b32 %0, %1" : "=v"(kwa[e]) : "v"(kq[u][e]));
        asm volatile("v_mov_b32 %0, %1" : "=v"(kwb[e]) : "v"(kq[u + 1][e]));
      }
#pragma unroll
      for (int i = 0; i < VWD; ++i) {
        asm volatile("v_mov_b32 %0, %1" : "=v"(vwa[i]) : "v"(vq[u][i]));
        asm volatile("v_mov_b32 %0, %1" : "=v"(vwb[i]) : "v"(vq[u + 1][i]));
      }
      float ka[EK], kb[EK], va[RPL], vb[RPL];
      widen_k(kwa, ka, BUF == 2 ? lane_value(ks_slot, j) : 1.f);
      widen_k(kwb, kb, BUF == 2 ? lane_value(ks_slot, j - 1) : 1.f);
      widen_v(vwa, va, BUF == 2 ? lane_value(vs_slot, j) : 1.f);
      widen_v(vwb, vb, BUF == 2 ? lane_value(vs_slot, j - 1) : 1.f);
      if (refill) {
        load_k(j - P, kq[u]);
        load_v(j - P, vq[u]);
        load_k(j - 1 - P, kq[u + 1]);
        load_v(j - 1 - P, vq[u + 1]);
      }
      float da = 0.f, db = 0.f, g = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) {
        da += ka[e] * yt[e];
        db += kb[e] * yt[e];
        g += ka[e] * kb[e];
      }
      wave_sum3_uniform(da, db, g);
      const float bta = lane_value(b_slot, j) * da;
      const float btb = lane_value(b_slot, j - 1) * (db - bta * g);
#pragma unroll
      for (int e = 0; e < EK; ++e) yt[e] = fmaf(-btb, kb[e], fmaf(-bta, ka[e], yt[e]));
      const float ca = bta * G;
      G *= lane_value(a_slot, j);
      const float cb = btb * G;
      G *= lane_value(a_slot, j - 1);
#pragma unroll
      for (int i = 0; i < RPL; ++i) acc[i] = fmaf(cb, vb[i], fmaf(ca, va[i], acc[i]));
    };
    static_assert(P % 2 == 0, "queue depth is even");
    int base = f - 1;
    for (; base >= CODE_LEAD * P - 1 && base >= P - 1; base -= P) {  // whole blocks: every slot is refilled
#pragma unroll
      for (int u = 0; u < P; u += 2) step2(u, base - u, true);
    }
    if constexpr (CODE_LEAD > 0) {  // at most CODE_LEAD blocks (plus the tail) before the rows are needed
      load_codes();
      grab();
    }
    for (; base >= P - 1; base -= P) {
#pragma unroll
      for (int u = 0; u < P; u += 2) step2(u, base - u, true);
    }
    // the last base + 1 < P writes are already in the queue: pairs, then one
#pragma unroll
    for (int u = 0; u + 1 < P; u += 2)
      if (u + 1 <= base) step2(u, base - u, false);
#pragma unroll
    for (int u = 0; u < P; u += 2)
      if (u == base) step(u, 0, false);
    if constexpr (CODE_LEAD == 0) {
      load_codes();
      grab();
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) wy[lane * EK + e] = G * yt[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // low-bit rows . y
    float d[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) d[i] = 0.f;
    constexpr int CPW = 32 / QB;  // codes per word
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
      const float4* y4 = reinterpret_cast<const float4*>(wy + CPU4 * c);
      float yy[CPU4];
#pragma unroll
      for (int q4 = 0; q4 < CPU4 / 4; ++q4) {
        const float4 t = y4[q4];
        yy[4 * q4] = t.x;
        yy[4 * q4 + 1] = t.y;
        yy[4 * q4 + 2] = t.z;
        yy[4 * q4 + 3] = t.w;
      }
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const uint32_t w[4] = {cw[i][c].x, cw[i][c].y, cw[i][c].z, cw[i][c].w};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int n = 0; n < CPW; ++n) d[i] = fmaf(code_at<QB>(w[q4], n), yy[CPW * q4 + n], d[i]);
      }
    }
    if constexpr (RPL == 2) {
      store_out2<OUT_BF16>(a.o, v_base + lane * 2, srow[0] * d[0] + acc[0], srow[1] * d[1] + acc[1]);
    } else {
      store_out<OUT_BF16>(a.o, v_base + lane, srow[0] * d[0] + acc[0]);
    }
    __builtin_amdgcn_wave_barrier();  // the next head reuses wy
    if (pooled) {  // pool index i: round r = 1 + i / 4, longest first within a round
      const int i = __builtin_amdgcn_readfirstlane(int(gv));
      const int r = 1 + (i >> 2), w = i & 3;
      o = r * NW + ((r & 1) ? NW - 4 - g4 + w : g4 + w);
    } else {
      ++k;
      o = k * NW + ((k & 1) ? NW - 1 - slot : slot);
    }
    if (o >= n_open) break;
    fetch(o);
  }
}

template <int DK, int DV, bool IN_BF16, bool OUT_BF16, bool WHT, int BUF, int QB>
__global__ __launch_bounds__(DEC_THREADS, DEC_WG_PER_CU) void decode_kernel(DecodeArgs a) {
  using S = DecShape<DK, DV>;
  constexpr int NT = S::NT;
  __shared__ float4 smem4[(S::L_END + 3) / 4];
  __shared__ uint64_t cmask[DEC_MAXB / 64];
  __shared__ int cpre[DEC_MAXB / 64 + 1];
  __shared__ uint8_t fills[DEC_MAXB];
  __shared__ uint16_t order[DEC_MAXB];
  __shared__ int vbase[64];
  __shared__ int pool_ctr;  // the open-head pool's next index
  extern __shared__ float4 dyn4[];  // buffered keys [W][DK]
  float* smem = reinterpret_cast<float*>(smem4);
  float* k_lds = reinterpret_cast<float*>(dyn4);
  float* x_lds = smem + S::L_X;
  float* y_lds = smem + S::L_Y;
  float* c_lds = smem + S::L_C;
  float* d_lds = smem + S::L_D;

  const int B = a.B, H = a.H, W = a.W;

  // ---- job list: which sequences close their window at this step
  const int nchunk = (B + 63) >> 6;
  if (threadIdx.x < 64) {
    for (int c = 0; c < nchunk; ++c) {
      const int s = c * 64 + threadIdx.x;
      int f = s < B ? a.fill_in[s] : 0;
      f = f < 0 ? 0 : (f > W - 1 ? W - 1 : f);  // out-of-range fill is a data error; stay in bounds
      if (s < B) fills[s] = uint8_t(f);
      const uint64_t m = __ballot(s < B && f == W - 1);
      if (threadIdx.x == 0) cmask[c] = m;
    }
    if (threadIdx.x == 0) {
      int acc = 0;
      for (int c = 0; c < nchunk; ++c) {
        cpre[c] = acc;
        acc += __popcll(cmask[c]);
      }
      cpre[nchunk] = acc;
    }
    // open sequences by fill, longest first, ties in sequence order (a
    // counting sort; every workgroup derives the same order).  vbase[v] is
    // first the count of open sequences at fill v, then the next position
    // for fill v.
    const int lane = threadIdx.x;
    vbase[lane] = 0;
    for (int c = 0; c < nchunk; ++c) {
      const int s = c * 64 + lane;
      const int f = s < B ? fills[s] : W - 1;
      if (f != W - 1) atomicAdd(&vbase[f], 1);
    }
    const float incl = wave_scan_incl(float(vbase[lane]));  // open sequences at fill <= lane (exact)
    const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
    vbase[lane] = int(total - incl);  // open sequences at a longer fill
    for (int c = 0; c < nchunk; ++c) {
      const int s = c * 64 + lane;
      const int f = s < B ? fills[s] : W - 1;
      const bool open = f != W - 1;
      uint64_t same = __ballot(open);  // lanes with an open sequence at this lane's fill
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        const uint64_t m = __ballot(open && ((f >> b) & 1));
        same &= ((f >> b) & 1) ? m : ~m;
      }
      const int r = __builtin_amdgcn_mbcnt_hi(uint32_t(same >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(same), 0));
      if (open) order[vbase[f] + r] = uint16_t(s);
      if (open && r == 0) vbase[f] += __popcll(same);
    }
  }
  if (threadIdx.x == 0) pool_ctr = 0;
  __syncthreads();
  JobList L;
  L.cmask = cmask;
  L.cpre = cpre;
  L.fills = fills;
  L.order = order;
  L.B = B;
  L.H = H;
  L.RC = S::RC;
  const int ncs = uniform(cpre[nchunk]);
  L.n_close_jobs = ncs * H * S::RC;
  L.n_jobs = L.n_close_jobs + (B - ncs) * H;

  // Roles: workgroups [0, OW) take the open heads, the rest the close jobs.
  // NW waves share the open heads (never more than there are heads); at
  // least one workgroup is left for close jobs when there are any.
  const int G = int(gridDim.x);
  const int n_open = L.n_jobs - L.n_close_jobs;
  int NW = a.open_waves < n_open ? a.open_waves : n_open;
  int OW = (NW + NT / 64 - 1) / (NT / 64);
  const int ow_max = L.n_close_jobs > 0 ? G - 1 : G;
  if (OW > ow_max) OW = ow_max;
  if (NW > OW * (NT / 64)) NW = OW * (NT / 64);
  int job = int(blockIdx.x) - OW;

  // ================================================================ close jobs
  // thread t: row rb*CR + t / CSEG, columns [(t % CSEG) * CCOL, +CCOL).  The
  // window's keys and this job's slice of its values are staged in LDS once;
  // each row then replays the W writes on its dequantized value in fp32,
  //   s <- alpha s + beta (v - alpha (s . k)) k,
  // where alpha s is formed while s . k is reduced, and the next write's key
  // and value are read from LDS while the current one is applied.
  for (; job >= 0 && job < L.n_close_jobs; job += G - OW) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // keep per-thread offsets from being hoisted out of the loop
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const JobId J = job_id(L, job);
    const int f = J.f;  // == W - 1
    const int bh = J.seq * H + J.h;
    const size_t qk_base = size_t(bh) * DK;
    const size_t v_base = size_t(bh) * DV;
    const size_t bufs_base = size_t(bh) * W;
    const int rr = tid / S::CSEG;
    const int seg = tid % S::CSEG;
    const int row = J.rb * S::CR + rr;
    const float alpha_t = a.alpha[bh];
    const float beta_t = a.beta[bh];
    RawVec<IN_BF16, S::EK> qraw, kraw;
    load_raw_vec<IN_BF16, S::EK>(a.q, qk_base + lane * S::EK, qraw);
    load_raw_vec<IN_BF16, S::EK>(a.k, qk_base + lane * S::EK, kraw);
    constexpr int EB = BUF == 0 ? 4 : BUF == 1 ? 2 : 1;  // bytes per buffered element
    const rsrc_t rk = make_rsrc(static_cast<const char*>(a.buf_k) + size_t(bh) * W * DK * EB, uint32_t(f) * DK * EB);
    // four consecutive buffered elements at element offset e0 (+ e1 scalar)
    // (E4M3: the codes; the caller applies the vector's scale)
    auto load4 = [&](const rsrc_t& r, uint32_t e0, uint32_t e1) __attribute__((always_inline)) {
      if constexpr (BUF == 1) {
        const uint2 w = bload_u2s<dec_pol(BUF)>(r, e0 * 2, e1 * 2);
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
      } else if constexpr (BUF == 2) {
        const uint32_t w = __float_as_uint(bload_f1s<dec_pol(BUF)>(r, e0, e1));
        const float2 lo = e4m3_unpack2(w, false), hi = e4m3_unpack2(w, true);
        return make_float4(lo.x, lo.y, hi.x, hi.y);
      } else {
        return bload_f4<dec_pol(BUF)>(r, e0 * 4, e1 * 4);
      }
    };
    // E4M3: the scale of slot j (slots past the fill read 0)
    auto slot_scale = [&](const float* sc, int j) __attribute__((always_inline)) {
      return bload_f1<dec_pol(BUF)>(make_rsrc(sc + bufs_base, uint32_t(f) * 4), uint32_t(j) * 4);
    };
    float4 kt[S::KREG];
#pragma unroll
    for (int i = 0; i < S::KREG; ++i) {
      kt[i] = load4(rk, uint32_t(tid) * 4, uint32_t(i * NT * 4));
      if constexpr (BUF == 2) {
        const float sc = slot_scale(a.ks, (tid * 4 + i * NT * 4) / DK);
        kt[i].x *= sc;
        kt[i].y *= sc;
        kt[i].z *= sc;
        kt[i].w *= sc;
      }
    }
    // lane j: alpha_j, beta_j of write j; the current token's in lane W - 1
    float a_slot = bload_f1<dec_pol(BUF)>(make_rsrc(a.buf_alpha + bufs_base, uint32_t(f) * 4), uint32_t(lane) * 4);
    float b_slot = bload_f1<dec_pol(BUF)>(make_rsrc(a.buf_beta + bufs_base, uint32_t(f) * 4), uint32_t(lane) * 4);
    // this thread's CCOL = 8 codes of its row (8 bytes, or 4 of 4-bit codes)
    uint2 cwr;
    if constexpr (QB == 8) {
      cwr = *reinterpret_cast<const uint2*>(a.codes + (v_base + row) * DK + seg * S::CCOL);
    } else {
      cwr.x = *reinterpret_cast<const uint32_t*>(a.codes + (v_base + row) * (DK / 2) + seg * (S::CCOL / 2));
      cwr.y = 0u;
    }
    const float srow = a.scales[v_base + row];
    const rsrc_t rv = make_rsrc(static_cast<const char*>(a.buf_v) + size_t(bh) * W * DV * EB, uint32_t(f) * DV * EB);
    float4 vt[S::CVREG];
#pragma unroll
    for (int i = 0; i < S::CVREG; ++i) {  // slot (tid + NT*i) / CVF4, rows 4*((tid + NT*i) % CVF4)
      vt[i] = load4(rv, uint32_t((tid / S::CVF4) * DV + (tid % S::CVF4) * 4),
                    uint32_t((i * NT / S::CVF4) * DV + J.rb * S::CR));
      if constexpr (BUF == 2) {
        const float sc = slot_scale(a.vs, tid / S::CVF4 + i * NT / S::CVF4);
        vt[i].x *= sc;
        vt[i].y *= sc;
        vt[i].z *= sc;
        vt[i].w *= sc;
      }
    }
    uint32_t vcur_raw = 0;
    if (tid < S::CR) vcur_raw = load_raw<IN_BF16>(a.v, v_base + J.rb * S::CR + tid);

    float qv[S::EK], kv[S::EK];
    unpack_raw_vec<IN_BF16, S::EK>(qraw, qv);
    unpack_raw_vec<IN_BF16, S::EK>(kraw, kv);
#pragma unroll
    for (int i = 0; i < S::KREG; ++i) {
      const int idx = tid + i * NT;
      if (idx < f * S::KF4) reinterpret_cast<float4*>(k_lds)[idx] = kt[i];
      consume(kt[i]);
    }
#pragma unroll
    for (int i = 0; i < S::CVREG; ++i) {
      const int idx = tid + i * NT;
      if (idx / S::CVF4 < f) reinterpret_cast<float4*>(x_lds)[idx] = vt[i];
    }
    if (tid < S::CR) x_lds[f * S::CR + tid] = raw_to_f32<IN_BF16>(vcur_raw);
    if (lane == f) {
      a_slot = alpha_t;
      b_slot = beta_t;
    }
    if constexpr (WHT) {
      fwht_group<S::EK, 64>(qv, lane);
      fwht_group<S::EK, 64>(kv, lane);
    }
    if (wave == 0) {  // the current token's key is the window's last write; q for the output
#pragma unroll
      for (int e = 0; e < S::EK; ++e) {
        k_lds[f * DK + lane * S::EK + e] = kv[e];
        y_lds[lane * S::EK + e] = qv[e];
      }
    }
    constexpr int CC = S::CCOL;
    float sv[CC];
    if constexpr (QB == 8) {
      const uint32_t w[2] = {cwr.x, cwr.y};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) sv[4 * h + c] = i8_at(w[h], c) * srow;
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) sv[c] = i4_at(cwr.x, c) * srow;
    }
    __syncthreads();  // keys and values staged
    auto read_kv = [&](int j, float (&kk)[CC], float& vv) __attribute__((always_inline)) {
      const float4* k4 = reinterpret_cast<const float4*>(k_lds + j * DK + seg * CC);
#pragma unroll
      for (int e = 0; e < CC / 4; ++e) {
        const float4 x = k4[e];
        kk[4 * e] = x.x;
        kk[4 * e + 1] = x.y;
        kk[4 * e + 2] = x.z;
        kk[4 * e + 3] = x.w;
      }
      vv = x_lds[j * S::CR + rr];
    };
    auto apply = [&](int j, const float (&kk)[CC], float vv) __attribute__((always_inline)) {
      const float aj = lane_value(a_slot, j);
      const float bj = lane_value(b_slot, j);
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int c = 0; c < CC; c += 2) {
        p0 = fmaf(sv[c], kk[c], p0);
        p1 = fmaf(sv[c + 1], kk[c + 1], p1);
      }
      const float sk = group_sum<S::CSEG>(p0 + p1);  // s . k_j
      const float coef = bj * fmaf(-aj, sk, vv);
#pragma unroll
      for (int c = 0; c < CC; ++c) sv[c] = fmaf(coef, kk[c], aj * sv[c]);
    };
    {
      float ka[CC], kb[CC], va, vb;
      read_kv(0, ka, va);
      int j = 0;
      for (; j + 2 <= W; j += 2) {  // the look-ahead reads are clamped into the window
        read_kv(j + 1, kb, vb);
        apply(j, ka, va);
        read_kv(min(j + 2, W - 1), ka, va);
        apply(j + 1, kb, vb);
      }
      if (j < W) apply(j, ka, va);
    }
    float po = 0.f, amax = 0.f;
#pragma unroll
    for (int c = 0; c < CC; ++c) {
      po += sv[c] * y_lds[seg * CC + c];
      amax = fmaxf(amax, fabsf(sv[c]));
    }
    po = group_sum<S::CSEG>(po);
    amax = group_max<S::CSEG>(amax);
    if constexpr (QB == 8) {
      const float scale = codec_scale(amax);
      uint2 wout;
      wout.x = pack4_i8(codec_code(sv[0], scale), codec_code(sv[1], scale), codec_code(sv[2], scale), codec_code(sv[3], scale));
      wout.y = pack4_i8(codec_code(sv[4], scale), codec_code(sv[5], scale), codec_code(sv[6], scale), codec_code(sv[7], scale));
      *reinterpret_cast<uint2*>(a.codes + (v_base + row) * DK + seg * CC) = wout;
      if (seg == 0) a.scales[v_base + row] = scale;
    } else {
      const float scale = codec_scale<7>(amax);
      int c4[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) c4[c] = codec_code<7>(sv[c], scale);
      *reinterpret_cast<uint32_t*>(a.codes + (v_base + row) * (DK / 2) + seg * (CC / 2)) = pack8_i4(c4);
      if (seg == 0) a.scales[v_base + row] = scale;
    }
    if (seg == 0) store_out<OUT_BF16>(a.o, v_base + row, po);
    if (tid == 0 && J.rb == 0 && J.h == 0) a.fill_out[J.seq] = 0;
    __syncthreads();  // LDS is reused by the next job
  }

  // ================================================================ open jobs
  // One wave per head at a time.  Taken longest window first, wave `slot`
  // gets positions slot, 2NW-1-slot, 2NW+slot, ... (a serpentine deal, so
  // every wave's total window length is about the same).  Fewer waves than
  // heads keeps the loads in flight near what saturates HBM, so the longest
  // windows are not starved behind the short ones.
  if (int(blockIdx.x) < OW) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int slot = int(blockIdx.x) * (NT / 64) + wave;
    float* wy = y_lds + wave * DK;
    if (slot < NW) open_wave<DK, DV, IN_BF16, OUT_BF16, WHT, BUF, QB>(a, L, slot, NW, n_open, lane, wy, &pool_ctr);
  }
}

// Schedule overrides (tuning and the schedule tests): the persistent grid
// size and the number of waves that take open heads, 0 = the defaults below.
// They start from GDNQ_DECODE_GRID / GDNQ_DECODE_OPEN_WAVES, read once when
// the library is loaded, and gdnq_decode_set_schedule replaces them.
struct DecodeSchedule {
  int grid, open_waves;
};
DecodeSchedule decode_schedule();

// Persistent grid: DEC_WG_PER_CU resident workgroups per CU on 256 CUs, never
// more workgroups than jobs.
inline unsigned decode_grid(int B, int H, int rc) {
  const long jobs_max = long(B) * H * rc;
  long g = 256 * DEC_WG_PER_CU;  // resident workgroups on 256 CUs
  const int o = decode_schedule().grid;
  if (o > 0) g = o;
  return unsigned(jobs_max < g ? jobs_max : g);
}

// Waves that take open heads.
inline int decode_open_waves() {
  const int o = decode_schedule().open_waves;
  return o > 0 ? o : DEC_OPEN_WAVES;
}

template <int DK, int DV, bool IB, bool OB, bool WHT, int BB, int QB>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const unsigned grid = decode_grid(a.B, a.H, DecShape<DK, DV>::RC);
  const size_t lds = size_t(a.W) * DK * sizeof(float);  // buffered keys
  hipLaunchKernelGGL((decode_kernel<DK, DV, IB, OB, WHT, BB, QB>), dim3(grid), dim3(DEC_THREADS), lds, s, a);
  return hipGetLastError();
}

template <int DK, int DV, int BB, int QB>
hipError_t launch_dkdv(const DecodeArgs& a, bool ib, bool ob, bool wht, hipStream_t s) {
  if (ib) {
    if (ob) return wht ? launch_t<DK, DV, true, true, true, BB, QB>(a, s) : launch_t<DK, DV, true, true, false, BB, QB>(a, s);
    return wht ? launch_t<DK, DV, true, false, true, BB, QB>(a, s) : launch_t<DK, DV, true, false, false, BB, QB>(a, s);
  }
  if (ob) return wht ? launch_t<DK, DV, false, true, true, BB, QB>(a, s) : launch_t<DK, DV, false, true, false, BB, QB>(a, s);
  return wht ? launch_t<DK, DV, false, false, true, BB, QB>(a, s) : launch_t<DK, DV, false, false, false, BB, QB>(a, s);
}

template <int BB, int QB>
hipError_t launch_bb(const DecodeLaunch& L, const DecodeArgs& a, hipStream_t stream) {
  if (L.d_k == 128 && L.d_v == 128) return launch_dkdv<128, 128, BB, QB>(a, L.in_bf16, L.out_bf16, L.wht, stream);
  if (L.d_k == 128 && L.d_v == 64) return launch_dkdv<128, 64, BB, QB>(a, L.in_bf16, L.out_bf16, L.wht, stream);
  if (L.d_k == 64 && L.d_v == 128) return launch_dkdv<64, 128, BB, QB>(a, L.in_bf16, L.out_bf16, L.wht, stream);
  return launch_dkdv<64, 64, BB, QB>(a, L.in_bf16, L.out_bf16, L.wht, stream);
}

template <int QB>
hipError_t launch_qb(const DecodeLaunch& L, const DecodeArgs& a, hipStream_t stream) {
  if (L.buf_fp8) return launch_bb<2, QB>(L, a, stream);
  return L.buf_bf16 ? launch_bb<1, QB>(L, a, stream) : launch_bb<0, QB>(L, a, stream);
}

// the 4-bit state's instantiations (decode_q4.hip)
hipError_t launch_decode_q4(const DecodeLaunch& L, const DecodeArgs& a, hipStream_t stream);

}  // namespace gdnq
