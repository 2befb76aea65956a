// Chunkwise-parallel prefill of the per-window int8-state gated delta rule
// on gfx950 ("LinQuant ...", abstract: chunkwise prefill as dense matrix
// products; "LeapQuant ...", abstract: requantize once per window).
//
// Chunk algebra (chunk of C = 64 tokens, state S0 at its start,
// g_i = sum_{s<=i} log alpha_s, gamma_i = exp(g_i)):
//   A_ij = beta_i exp(g_i - g_j) k_i.k_j  (j < i),   T = (I + A)^-1
//   U    = T (diag(beta) V - diag(beta gamma) K S0^T)
//   O    = diag(gamma) Q S0^T + (L o Q K^T) U,        L_ij = exp(g_i - g_j), j <= i
//   S_C  = gamma_C S0 + U^T diag(exp(g_C - g)) K
// With the window equal to the chunk, S0 is always a dequantized state
// (codes * row scale) and S_C is requantized at every chunk end.  A last
// chunk of r < 64 tokens (a sequence handed over to decode with its window
// still open) is padded with k = 0, alpha = 1, beta = 0, which leaves T's
// valid block, U and O of the valid tokens unchanged; its state update and
// requantization are skipped, so the stored state stays at the last window
// boundary.
//
// Two kernels:
//   prep  -- one workgroup per chunk-head, all in parallel: K K^T on bf16
//            MFMA (bf16 inputs, exact products), A, and T by blocked forward
//            substitution (diagonal 16x16 blocks on the VALU, off-diagonal
//            blocks on fp32 MFMA); T (as three bf16 parts) and g go to the
//            workspace.
//   state -- one workgroup per (sequence, head, block of 32 rows): rows of
//            the state evolve independently, so each workgroup carries its
//            rows (codes + scales in LDS) through all chunks, four barriers
//            per chunk, the next chunk's inputs prefetched into registers.
//            Every product runs on bf16 MFMA: K S0^T and Q S0^T take the codes
//            exactly; T (rhs), (U o d)^T K and M U split their fp32 operands
//            into two or three bf16 parts, which keeps fp32-level accuracy.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "mfma.h"

namespace gdnq {

constexpr int PC = 64;    // chunk = window
constexpr int PD = 128;   // d_k = d_v
constexpr int RWS = 32;   // state rows per state-pass workgroup

__device__ __forceinline__ void tile_of(int tt, int& it, int& jt) {
  it = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;  // lower 16x16 tiles (it >= jt), row-major
  jt = tt - it * (it + 1) / 2;
}

// exp for the output-only decay factors (arguments <= 0): one v_exp_f32,
// relative error ~1e-6, far inside the output tolerance
__device__ __forceinline__ float exp_out(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Where sequence b's tokens and chunks are.  A sequence is the pre_b writes
// that decode still holds in its window buffer (when resuming; none
// otherwise) followed by its n_b new tokens, and its chunks of 64 run over
// that whole sequence from its first buffered write: chunk 0 is the window
// that is still open.  Uniform: n_b = T, no prefix, nothing mapped.  Mapped
// (variable lengths or resuming): the workspace's sanitized token offsets
// tok[0..B], prefix lengths pre[0..B) and chunk offsets ch[0..B].  When
// resuming, chunk 0 of every sequence (prefix and first new tokens) is read
// from a staged copy laid out like the tokens ([B][64][H][...]).
struct SeqMap {
  const int32_t* tok;  // nullptr: uniform
  const int32_t* ch;
  const int32_t* pre;  // nullptr: no prefix, nothing staged
  const uint16_t* sk;  // staged chunk 0: k, q, v (bf16) and alpha, beta
  const uint16_t* sq;
  const uint16_t* sv;
  const float* sa;
  const float* sb;
  const int32_t* order;  // sequences by chunk count, most first (nullptr: in order)
  int T;               // tokens per sequence (uniform) or in total
  __device__ size_t tok0(int b) const { return tok ? size_t(tok[b]) : size_t(b) * T; }
  __device__ int ntok(int b) const { return tok ? tok[b + 1] - tok[b] : T; }
  __device__ int npre(int b) const { return pre ? pre[b] : 0; }
  __device__ int len(int b) const { return npre(b) + ntok(b); }
  __device__ int chunk0(int b) const { return tok ? ch[b] : b * ((T + 63) / 64); }
  __device__ bool staged(int c) const { return pre != nullptr && c == 0; }
  // row of position c * 64 in its source: the staged copy, or the tokens
  __device__ size_t row0(int b, int c) const {
    return staged(c) ? size_t(b) * 64 : tok0(b) + size_t(c) * 64 - size_t(npre(b));
  }
};

// ---------------------------------------------------------------- prep
constexpr int KP = 136;  // bf16 pitch of [token][dim] tiles
constexpr int AP = 65;   // fp32 pitch of A
constexpr int PREP_GRID = 4 * 256;  // prep workgroups: four per CU
constexpr int PREP_KT = PC * KP * 2 > (PC * PC + 3 * 256) * 4 ? PC * KP * 2 : (PC * PC + 3 * 256) * 4;

struct PrepArgs {
  const uint16_t* k;
  const float* alpha;
  const float* beta;
  __bf16* T_ws;  // [chunks*H][3][64][64]: T as hi/mid/lo bf16 planes
  float* g_ws;  // [chunks*H][64]
  SeqMap sm;
  int B, H;
  int total;  // chunk-heads the grid covers (an upper bound when mapped)
};

__global__ __launch_bounds__(256) void gdn_prep_kernel(PrepArgs a) {
  // K is only needed for K K^T; T and the level products reuse its space
  __shared__ __attribute__((aligned(16))) unsigned char kt_raw[PREP_KT];
  __shared__ float Al[PC * AP];
  __shared__ float gl[PC], bl[PC];
  __bf16* Kl = reinterpret_cast<__bf16*>(kt_raw);
  float* Tl = reinterpret_cast<float*>(kt_raw);
  float* Pl = Tl + PC * PC;
  // Each workgroup takes chunk-heads blockIdx.x, + gridDim.x, ... (index
  // chunk * H + h, chunks numbered across the sequences) and loads the next
  // one's keys, alpha and beta into registers while it works on the current.
  struct Src {
    const uint16_t* k;
    const float* al;
    const float* be;
    size_t tok0;  // row of the chunk's first position in its source
    int h, nvalid;  // tokens of the chunk in the sequence (< 64 only in a last, partial chunk)
    bool ok;
  };
  auto locate = [&](int idx) {
    Src r{};
    r.ok = idx < a.total;
    if (!r.ok) return r;
    r.h = idx % a.H;
    const int g = idx / a.H;
    int b;
    if (a.sm.tok) {  // mapped: the chunk count is only bounded by the grid
      if (g >= a.sm.ch[a.B]) {
        r.ok = false;
        return r;
      }
      int lo = 0, hi = a.B - 1;  // last b with ch[b] <= g
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.sm.ch[mid] <= g) lo = mid; else hi = mid - 1;
      }
      b = lo;
    } else {
      b = g / ((a.sm.T + PC - 1) / PC);
    }
    const int c = g - a.sm.chunk0(b);
    r.tok0 = a.sm.row0(b, c);
    const bool stg = a.sm.staged(c);
    r.k = stg ? a.sm.sk : a.k;
    r.al = stg ? a.sm.sa : a.alpha;
    r.be = stg ? a.sm.sb : a.beta;
    r.nvalid = a.sm.len(b) - c * PC;
    return r;
  };
  // keys: thread -> token tid / 4, dims [(tid % 4) * 32, +32); padding keys
  // are 0.  alpha, beta: thread tid < 64 -> token tid (padding: 1 and 0).
  uint4 w[4];
  float al_t = 1.f, be_t = 0.f;
  auto load = [&](const Src& r) {
    const int tid = threadIdx.x;
    const int i = tid >> 2, qq = tid & 3;
    const int ic = i < r.nvalid ? i : r.nvalid - 1;
    const uint4* src = reinterpret_cast<const uint4*>(r.k + ((r.tok0 + ic) * a.H + r.h) * PD + qq * 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = i < r.nvalid ? src[e] : make_uint4(0u, 0u, 0u, 0u);
    if (tid < 64) {
      const size_t t = (r.tok0 + (tid < r.nvalid ? tid : r.nvalid - 1)) * a.H + r.h;
      al_t = tid < r.nvalid ? r.al[t] : 1.f;
      be_t = tid < r.nvalid ? r.be[t] : 0.f;
    }
  };
  int idx = blockIdx.x;
  Src cur = locate(idx);
  if (!cur.ok) return;
  load(cur);
  for (;;) {
  // per-thread offsets recomputed each round: hoisted out of the loop, the
  // LDS addresses of the unrolled products would hold ~130 registers
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  {
    const int i = tid >> 2, qq = tid & 3;
    uint4* dst = reinterpret_cast<uint4*>(Kl + i * KP + qq * 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = w[e];
  }
  if (tid < 64) {  // g = inclusive prefix sum of log alpha
    float la = logf(al_t);
    bl[tid] = be_t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const float o = __shfl_up(la, s, 64);
      if (lane >= s) la += o;
    }
    gl[tid] = la;
    a.g_ws[size_t(idx) * PC + tid] = la;
  }
  // the next chunk-head's loads fly during this one's work
  const int nidx = idx + int(gridDim.x);
  const Src nxt = locate(nidx);
  if (nxt.ok) load(nxt);
  __syncthreads();

  // A from the lower 16x16 tiles of K K^T (kept in registers until K is dead)
  float av[3][4];
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    const int tt = wave + 4 * n;
    if (tt < 10) {
      int it, jt;
      tile_of(tt, it, jt);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        acc = mfma16(lds_bf16x8(Kl + (it * 16 + lr) * KP + kk), lds_bf16x8(Kl + (jt * 16 + lr) * KP + kk), acc);
      }
      const int j = jt * 16 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = it * 16 + 4 * lq + q;
        av[n][q] = (j < i) ? bl[i] * expf(gl[i] - gl[j]) * acc[q] : 0.f;
      }
    }
  }
  __syncthreads();  // K dead from here; its space becomes T
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    const int tt = wave + 4 * n;
    if (tt < 10) {
      int it, jt;
      tile_of(tt, it, jt);
#pragma unroll
      for (int q = 0; q < 4; ++q) Al[(it * 16 + 4 * lq + q) * AP + jt * 16 + lr] = av[n][q];
    }
  }
  // strictly upper blocks of T are zero
  for (int e = tid; e < 6 * 256; e += 256) {
    const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    const int bi = blk < 3 ? 0 : blk < 5 ? 1 : 2;
    const int bj = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
    Tl[(bi * 16 + rr) * PC + bj * 16 + cc] = 0.f;
  }
  __syncthreads();

  // diagonal 16x16 blocks of T: forward substitution, one column per lane
  if (wave == 0) {
    const int bb = lane >> 4, cc = lane & 15;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) s -= Al[(bb * 16 + r) * AP + bb * 16 + j] * t[j];
      t[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tl[(bb * 16 + r) * PC + bb * 16 + cc] = t[r];
  }
  __syncthreads();

  // off-diagonal blocks, one block-diagonal at a time (fp32 MFMA):
  //   P = sum_{k=j}^{i-1} A_ik T_kj,   T_ij = -T_ii P
  for (int d = 1; d <= 3; ++d) {
    const int nb = 4 - d;
    if (wave < nb) {
      const int i = d + wave, j = wave;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = j; kb < i; ++kb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma4(Al[(i * 16 + lr) * AP + kb * 16 + 4 * kk + lq], Tl[(kb * 16 + 4 * kk + lq) * PC + j * 16 + lr], acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) Pl[wave * 256 + (4 * lq + q) * 16 + lr] = acc[q];
    }
    __syncthreads();
    if (wave < nb) {
      const int i = d + wave, j = wave;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma4(Tl[(i * 16 + lr) * PC + i * 16 + 4 * kk + lq], Pl[wave * 256 + (4 * kk + lq) * 16 + lr], acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) Tl[(i * 16 + 4 * lq + q) * PC + j * 16 + lr] = -acc[q];
    }
    __syncthreads();
  }

  {  // T as three bf16 planes: thread -> row tid / 4, columns [(tid % 4) * 16, +16)
    const int i = tid >> 2, c0 = (tid & 3) * 16;
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 t4 = *reinterpret_cast<const float4*>(Tl + i * PC + c0 + e);
      x[e] = t4.x;
      x[e + 1] = t4.y;
      x[e + 2] = t4.z;
      x[e + 3] = t4.w;
    }
    bf16x8 p[3][2];
    {
      float lo8[8], hi8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo8[e] = x[e];
        hi8[e] = x[8 + e];
      }
      split3(lo8, p[0][0], p[1][0], p[2][0]);
      split3(hi8, p[0][1], p[1][1], p[2][1]);
    }
    __bf16* dst = a.T_ws + size_t(idx) * 3 * PC * PC + i * PC + c0;
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
      *reinterpret_cast<bf16x8*>(dst + pl * PC * PC) = p[pl][0];
      *reinterpret_cast<bf16x8*>(dst + pl * PC * PC + 8) = p[pl][1];
    }
  }
  if (!nxt.ok) break;
  idx = nidx;
  cur = nxt;
  __syncthreads();  // the next chunk's keys overwrite T's space
  }
}

// ---------------------------------------------------------------- state pass
struct StateArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* beta;
  const __bf16* T_ws;
  const float* g_ws;
  const int8_t* init_codes;
  const float* init_scales;
  void* o;
  int8_t* codes;
  float* scales;
  SeqMap sm;
  int B, H;
};

constexpr int TP = 72;    // bf16 pitch of [64][64] planes (T, M) and [32][64] planes (rhs^T, U^T)
constexpr int SNP = 132;  // fp32 pitch of the new rows [32][128]
constexpr int CBP = 136;  // bf16 pitch of the codes [32][128]

// LDS carve (bytes)
constexpr int OFF_K = 0;                           // K  [64][KP] bf16
constexpr int OFF_Q = OFF_K + PC * KP * 2;         // Q  [64][KP] bf16
constexpr int OFF_KT = OFF_Q + PC * KP * 2;        // K^T [128][64] bf16, 16-byte granules xor-swizzled
constexpr int OFF_T = OFF_KT + PD * PC * 2;        // T   hi/mid/lo [3][64][TP] bf16
constexpr int OFF_M = OFF_T + 3 * PC * TP * 2;     // M   hi/lo [2][64][TP] bf16
constexpr int OFF_R = OFF_M + 2 * PC * TP * 2;     // rhs^T hi/mid/lo [3][32][TP] bf16 (plane 0 holds V^T until rhs)
constexpr int OFF_UD = OFF_R + 3 * RWS * TP * 2;   // (U o d)^T hi/mid/lo [3][32][TP] bf16
constexpr int OFF_U = OFF_UD + 3 * RWS * TP * 2;   // U^T hi/lo [2][32][TP] bf16
constexpr int OFF_SN = OFF_U + 2 * RWS * TP * 2;   // new rows [32][SNP] fp32
constexpr int OFF_CB = OFF_SN + RWS * SNP * 4;     // codes [32][CBP] bf16 (exact)
constexpr int OFF_G = OFF_CB + RWS * CBP * 2;      // per chunk parity: g, exp(g), beta [2][3][64]
constexpr int OFF_D = OFF_G + 2 * 3 * PC * 4;      // exp(g_C - g) [64], row scales [32]
constexpr int STATE_LDS = OFF_D + (PC + RWS) * 4;
static_assert(STATE_LDS <= 160 * 1024, "state-pass LDS");

__device__ __forceinline__ int kt_index(int d, int j) {  // bf16 index of K^T[d][j]
  return d * PC + ((((j >> 3) ^ (d >> 3)) & 7) << 3) + (j & 7);
}

__device__ __forceinline__ uint2 as_u2(const bf16x4& v) { return __builtin_bit_cast(uint2, v); }

// Per chunk the state pass runs four phases between barriers, on two roles:
//   eight chain waves (the recurrence itself)      eight side waves
//   A  X = K S0^T; rhs                             Q S0^T, scaled: output base
//   B  U = T rhs; U^T and (U o d)^T parts          stage K, Q of the next chunk; load two ahead
//   C  S_C^T = gamma_C S0^T + K^T (U o d)          O = base + M U; stage T, V, g, beta of the
//                                                  next chunk; load two ahead
//   D  requantize S_C (and two tiles of M)         next chunk's K^T and M = L o Q K^T
// Everything the recurrence does not wait on (the output, staging, memory
// traffic, the next chunk's K^T and M) runs on the side waves, so a phase
// lasts as long as the longer of the two roles' work, not their sum.  Every
// prefetched register is consumed one chunk after it is loaded.
constexpr int SNT = 1024;   // state-pass threads
constexpr int NCRIT = 512;  // threads of the chain waves

// QB: the state's code width, 8 (int8) or 4 (packed 4-bit, scale absmax / 7)
template <bool OUT_BF16, int QB>
__global__ __launch_bounds__(SNT, 1) void gdn_state_kernel(StateArgs a) {
  constexpr int QMAX = QB == 8 ? 127 : 7;
  constexpr int RB = PD * QB / 8;  // bytes per stored row
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __bf16* Kl = reinterpret_cast<__bf16*>(lds + OFF_K);
  __bf16* Ql = reinterpret_cast<__bf16*>(lds + OFF_Q);
  __bf16* KT = reinterpret_cast<__bf16*>(lds + OFF_KT);
  __bf16* Tp = reinterpret_cast<__bf16*>(lds + OFF_T);
  __bf16* Mp = reinterpret_cast<__bf16*>(lds + OFF_M);
  __bf16* Rp = reinterpret_cast<__bf16*>(lds + OFF_R);
  __bf16* Dp = reinterpret_cast<__bf16*>(lds + OFF_UD);
  __bf16* Up = reinterpret_cast<__bf16*>(lds + OFF_U);
  float* Sn = reinterpret_cast<float*>(lds + OFF_SN);
  __bf16* Cb = reinterpret_cast<__bf16*>(lds + OFF_CB);
  float* G = reinterpret_cast<float*>(lds + OFF_G);  // parity p: g at G + 192 p, exp(g) +64, beta +128
  float* dl = reinterpret_cast<float*>(lds + OFF_D);
  float* sl = dl + PC;

  const int nblk = a.B * a.H * (PD / RWS);
  const int logical = xcd_swizzle(blockIdx.x, nblk);  // the 4 row blocks of a head share an XCD
  const int chain = logical / (PD / RWS);
  const int rb = logical % (PD / RWS);
  // With a length order, the chains go round robin over the eight XCD
  // segments of the swizzle, so every XCD takes its share longest first
  // (a contiguous slice of the order would give one XCD all the long ones).
  int cr = chain;
  if (a.sm.order && (nblk & 31) == 0) {
    const int seg = nblk >> 5;  // chains per XCD segment
    cr = (chain % seg) * 8 + chain / seg;
  }
  const int b = a.sm.order && (nblk & 31) == 0 ? a.sm.order[cr / a.H] : chain / a.H;
  const int h = cr % a.H;
  const int r0 = rb * RWS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int Tb = a.sm.len(b);  // this sequence's positions (buffered prefix and new tokens)
  const int NC = (Tb + PC - 1) / PC;
  const bool partial_last = (Tb % PC) != 0;  // the last chunk holds fewer than 64 tokens
  const size_t HD = size_t(a.H) * PD;
  const size_t state_row0 = (size_t(b) * a.H + h) * PD + r0;
  const size_t tokb = a.sm.tok0(b);

  // one 16x16 tile of M = L o Q K^T of the staged chunk: tiles 0..9 are the
  // lower tiles, D[j][i] = k_j . q_i stored as M[i][j] (hi and lo parts);
  // tiles 10 and 11 the two zero tiles above the diagonal that the 32-token
  // steps of M U reach
  auto build_m_tile = [&](int tt, const float* gc) __attribute__((always_inline)) {
    int mi, mj;
    float m4[4] = {0.f, 0.f, 0.f, 0.f};
    if (tt < 10) {
      tile_of(tt, mi, mj);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        acc = mfma16(lds_bf16x8(Kl + (mj * 16 + lr) * KP + kk), lds_bf16x8(Ql + (mi * 16 + lr) * KP + kk), acc);
      }
      const int i = mi * 16 + lr;
      const float gi = gc[i];
      const float4 g4 = *reinterpret_cast<const float4*>(gc + mj * 16 + 4 * lq);
      const float gj[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = mj * 16 + 4 * lq + q;
        m4[q] = (j <= i) ? exp_out(gi - gj[q]) * acc[q] : 0.f;
      }
    } else {
      mi = tt == 10 ? 0 : 2;
      mj = mi + 1;
    }
    bf16x4 h1, h2;
    split2(m4, h1, h2);
    const int i = mi * 16 + lr, j0 = mj * 16 + 4 * lq;
    *reinterpret_cast<uint2*>(Mp + i * TP + j0) = as_u2(h1);
    *reinterpret_cast<uint2*>(Mp + PC * TP + i * TP + j0) = as_u2(h2);
  };

  if (tid < NCRIT) {
    // ================================================================ chain waves
    const int it = wave >> 1, rt = wave & 1;  // this wave's (token tile, row tile) of X and U
    const int nks = (it >> 1) + 1;            // 32-token steps reaching the diagonal of tile it
    const int r = rt * 16 + lr;
    const int i0 = it * 16 + 4 * lq;
    {  // stored rows at the start (zero state without init)
      const int rq = tid >> 4, seg = tid & 15;  // 32 rows x 16 segments of 8 codes
      bf16x8 cv;
      if constexpr (QB == 8) {
        uint2 w = make_uint2(0u, 0u);
        if (a.init_codes) w = *reinterpret_cast<const uint2*>(a.init_codes + (state_row0 + rq) * RB + seg * 8);
        cv = i8x8_to_bf16(w);
      } else {
        uint32_t w = 0u;
        if (a.init_codes) w = *reinterpret_cast<const uint32_t*>(a.init_codes + (state_row0 + rq) * RB + seg * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) cv[e] = (__bf16)i4_at(w, e);
      }
      *reinterpret_cast<bf16x8*>(Cb + rq * CBP + seg * 8) = cv;
      if (seg == 0) sl[rq] = a.init_scales ? a.init_scales[state_row0 + rq] : 0.f;
    }
    if (NC > 0) {
      __syncthreads();  // the side waves stage chunk 0
      if (wave < 2) build_m_tile(8 + wave, G);
    }
    __syncthreads();  // ... and build its K^T and the rest of M

    for (int c = 0; c < NC; ++c) {
      const float* gc = G + 192 * (c & 1);
      // ---- A: X = K S0^T (codes exact), rhs
      {
        f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kk = ks * 32 + 8 * lq;
          xacc = mfma16(lds_bf16x8(Kl + (it * 16 + lr) * KP + kk), lds_bf16x8(Cb + r * CBP + kk), xacc);
        }
        const float sr = sl[r];
        const float4 e4 = *reinterpret_cast<const float4*>(gc + 64 + i0);
        const float4 b4 = *reinterpret_cast<const float4*>(gc + 128 + i0);
        const float ge[4] = {e4.x, e4.y, e4.z, e4.w}, be[4] = {b4.x, b4.y, b4.z, b4.w};
        const uint2 vw = *reinterpret_cast<const uint2*>(Rp + r * TP + i0);
        const float vv[4] = {__uint_as_float(vw.x << 16), __uint_as_float(vw.x & 0xffff0000u),
                             __uint_as_float(vw.y << 16), __uint_as_float(vw.y & 0xffff0000u)};
        float rh[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) rh[q] = be[q] * (vv[q] - ge[q] * (sr * xacc[q]));
        bf16x4 h1, h2, h3;
        split3(rh, h1, h2, h3);
        *reinterpret_cast<uint2*>(Rp + r * TP + i0) = as_u2(h1);
        *reinterpret_cast<uint2*>(Rp + RWS * TP + r * TP + i0) = as_u2(h2);
        *reinterpret_cast<uint2*>(Rp + 2 * RWS * TP + r * TP + i0) = as_u2(h3);
      }
      if (tid < 64) dl[tid] = expf(gc[PC - 1] - gc[tid]);
      __syncthreads();

      // ---- B: U = T rhs (T unit lower triangular; six split products), then
      //      U^T (two parts) and (U o d)^T (three parts)
      {
        f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ub = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < nks; ++ks) {
          const int kk = ks * 32 + 8 * lq;
          const __bf16* tr = Tp + (it * 16 + lr) * TP + kk;
          const __bf16* rr = Rp + r * TP + kk;
          const bf16x8 t1 = lds_bf16x8(tr), t2 = lds_bf16x8(tr + PC * TP), t3 = lds_bf16x8(tr + 2 * PC * TP);
          const bf16x8 b1 = lds_bf16x8(rr), b2 = lds_bf16x8(rr + RWS * TP), b3 = lds_bf16x8(rr + 2 * RWS * TP);
          ua = mfma16(t2, b2, ua);
          ub = mfma16(t3, b1, ub);
          ua = mfma16(t1, b3, ua);
          ub = mfma16(t2, b1, ub);
          ua = mfma16(t1, b2, ua);
          ub = mfma16(t1, b1, ub);
        }
        const float4 d4 = *reinterpret_cast<const float4*>(dl + i0);
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
        float u[4], ud[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u[q] = ua[q] + ub[q];
          ud[q] = u[q] * dd[q];
        }
        bf16x4 h1, h2, h3;
        split2(u, h1, h2);
        *reinterpret_cast<uint2*>(Up + r * TP + i0) = as_u2(h1);
        *reinterpret_cast<uint2*>(Up + RWS * TP + r * TP + i0) = as_u2(h2);
        split3(ud, h1, h2, h3);
        *reinterpret_cast<uint2*>(Dp + r * TP + i0) = as_u2(h1);
        *reinterpret_cast<uint2*>(Dp + RWS * TP + r * TP + i0) = as_u2(h2);
        *reinterpret_cast<uint2*>(Dp + 2 * RWS * TP + r * TP + i0) = as_u2(h3);
      }
      __syncthreads();

      // ---- C: new rows S_C^T = gamma_C S0^T + K^T (U o d) (not for a partial last chunk:
      //      its window stays open and the stored state stays at the last boundary)
      const bool update = !(partial_last && c == NC - 1);
      if (update) {
        const int dt0 = (wave >> 1) * 2;
        bf16x8 u1[2], u2[2], u3[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const __bf16* dp = Dp + r * TP + ks * 32 + 8 * lq;
          u1[ks] = lds_bf16x8(dp);
          u2[ks] = lds_bf16x8(dp + RWS * TP);
          u3[ks] = lds_bf16x8(dp + 2 * RWS * TP);
        }
        const float gs = gc[64 + PC - 1] * sl[r];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int dt = dt0 + cc;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 ak = lds_bf16x8(KT + kt_index(dt * 16 + lr, ks * 32 + 8 * lq));
            acc = mfma16(ak, u3[ks], acc);
            acc = mfma16(ak, u2[ks], acc);
            acc = mfma16(ak, u1[ks], acc);
          }
          const int d0 = dt * 16 + 4 * lq;
          const bf16x4 c4 = *reinterpret_cast<const bf16x4*>(Cb + r * CBP + d0);
          float4 sn;
          sn.x = gs * float(c4[0]) + acc[0];
          sn.y = gs * float(c4[1]) + acc[1];
          sn.z = gs * float(c4[2]) + acc[2];
          sn.w = gs * float(c4[3]) + acc[3];
          *reinterpret_cast<float4*>(Sn + r * SNP + d0) = sn;
        }
      }
      __syncthreads();

      // ---- D: requantize the new rows
      if (update) {
        const int rq = tid >> 4, seg = tid & 15;
        const float4 s0 = *reinterpret_cast<const float4*>(Sn + rq * SNP + seg * 8);
        const float4 s1 = *reinterpret_cast<const float4*>(Sn + rq * SNP + seg * 8 + 4);
        const float x[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
        amax = group_max<16>(amax);
        const float scale = codec_scale<QMAX>(amax);
        float cf[8];
        codec_codes<8, QMAX>(x, scale, cf);
        bf16x8 cv;
#pragma unroll
        for (int e = 0; e < 8; ++e) cv[e] = (__bf16)cf[e];
        *reinterpret_cast<bf16x8*>(Cb + rq * CBP + seg * 8) = cv;
        if (seg == 0) sl[rq] = scale;
      }
      if (wave < 2 && c + 1 < NC) build_m_tile(8 + wave, G + 192 * ((c + 1) & 1));
      __syncthreads();
    }

    {  // final rows (codes back to int8, or packed 4-bit)
      const int rq = tid >> 4, seg = tid & 15;
      const bf16x8 cv = lds_bf16x8(Cb + rq * CBP + seg * 8);
      if constexpr (QB == 8) {
        uint2 w;
        w.x = pack4_i8(int(float(cv[0])), int(float(cv[1])), int(float(cv[2])), int(float(cv[3])));
        w.y = pack4_i8(int(float(cv[4])), int(float(cv[5])), int(float(cv[6])), int(float(cv[7])));
        *reinterpret_cast<uint2*>(a.codes + (state_row0 + rq) * RB + seg * 8) = w;
      } else {
        int c4[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c4[e] = int(float(cv[e]));
        *reinterpret_cast<uint32_t*>(a.codes + (state_row0 + rq) * RB + seg * 4) = pack8_i4(c4);
      }
      if (seg == 0) a.scales[state_row0 + rq] = sl[rq];
    }
    return;
  }

  // ================================================================ side waves
  const int st = tid - NCRIT;  // 0 .. 511
  const int sw = st >> 6;      // side wave 0 .. 7: the chain wave whose (token tile, row tile) it outputs
  // load mapping: K/Q token pair pm, dims [8 ps, +8); T row ti, columns
  // [8 tc, +8) of each plane; V for chain lane st, in its MFMA output layout
  const int pm = st & 31, ps = st >> 5;
  const int ti = st >> 3, tc = st & 7;
  const int vr = (sw & 1) * 16 + lr, vi = (sw >> 1) * 16 + 4 * lq;
  const size_t kq_off = size_t(h) * PD + 8 * ps, v_off = size_t(h) * PD + r0 + vr;
  const size_t wsc = size_t(a.sm.chunk0(b)) * a.H + h;  // workspace index of the first chunk
  const __bf16* tb = a.T_ws + wsc * 3 * PC * PC + ti * PC + 8 * tc;
  const float* gb = a.g_ws + wsc * PC + (st & 63);
  const size_t ch_step = size_t(a.H) * 3 * PC * PC;  // T elements per chunk (all heads)
  // position i of chunk c: whether it is in the sequence, and the row the
  // loads read (clamped into the sequence; padding is zeroed when staged)
  // the sequence map is read once, here: in the loop a scalar load's wait
  // would also wait for every LDS access in flight
  const int npre = a.sm.npre(b);
  const bool stg0 = a.sm.pre != nullptr;  // chunk 0 is read from the staged copy
  const size_t row_c0 = stg0 ? size_t(b) * PC : tokb;
  const size_t row_t = tokb - size_t(npre);  // chunk c >= 1 starts at row row_t + 64 c (wraps back for c >= 1)
  const uint16_t* const k_c0 = stg0 ? a.sm.sk : a.k;
  const uint16_t* const q_c0 = stg0 ? a.sm.sq : a.q;
  const uint16_t* const v_c0 = stg0 ? a.sm.sv : a.v;
  const float* const b_c0 = stg0 ? a.sm.sb : a.beta;
  const uint32_t HD32 = uint32_t(HD);
  auto tok_ok = [&](int c, int i) { return c * PC + i < Tb; };
  // chunk c's first row (scalar, 64-bit) and the in-chunk row a lane reads
  // (32-bit, clamped into the sequence)
  auto chunk_row = [&](int c) { return c == 0 ? row_c0 : row_t + size_t(c) * PC; };
  auto in_row = [&](int c, int i) {
    const int lim = Tb - 1 - c * PC;
    return uint32_t(i < lim ? i : lim);
  };
  int kq_c = 0, tv_c = 0;  // the chunks the prefetch registers hold

  // (clang vector types: arrays of HIP's uint4 are copied through memory)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 k0, k1, q0, q1;  // K, Q of the next chunk (or the one after)
  u32x4 t0, t1, t2;      // T parts, V, g, beta likewise
  uint32_t v4[4];
  float gv = 0.f, bv = 0.f;
  auto load_kq = [&](int c) {
    kq_c = c;
    const size_t cr = chunk_row(c) * HD + kq_off;
    const uint16_t* kb = (c == 0 ? k_c0 : a.k) + cr;
    const uint16_t* qb = (c == 0 ? q_c0 : a.q) + cr;
    const uint32_t o0 = in_row(c, 2 * pm) * HD32, o1 = in_row(c, 2 * pm + 1) * HD32;
    k0 = *reinterpret_cast<const u32x4*>(kb + o0);
    k1 = *reinterpret_cast<const u32x4*>(kb + o1);
    q0 = *reinterpret_cast<const u32x4*>(qb + o0);
    q1 = *reinterpret_cast<const u32x4*>(qb + o1);
  };
  auto load_tv = [&](int c) {
    tv_c = c;
    const __bf16* tp = tb + size_t(c) * ch_step;
    t0 = *reinterpret_cast<const u32x4*>(tp);
    t1 = *reinterpret_cast<const u32x4*>(tp + PC * PC);
    t2 = *reinterpret_cast<const u32x4*>(tp + 2 * PC * PC);
    const size_t cr = chunk_row(c);
    const uint16_t* vb = (c == 0 ? v_c0 : a.v) + cr * HD + v_off;
    const float* bb = (c == 0 ? b_c0 : a.beta) + cr * a.H + h;
#pragma unroll
    for (int q = 0; q < 4; ++q) v4[q] = vb[in_row(c, vi + q) * HD32];
    gv = gb[size_t(c) * a.H * PC];  // every side lane loads (one wave's worth is used): no branch
    bv = bb[in_row(c, st & 63) * uint32_t(a.H)];
  };
  auto stage_kq = [&]() {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool ok0 = tok_ok(kq_c, 2 * pm), ok1 = tok_ok(kq_c, 2 * pm + 1);
    *reinterpret_cast<u32x4*>(Kl + (2 * pm) * KP + 8 * ps) = ok0 ? k0 : z;
    *reinterpret_cast<u32x4*>(Kl + (2 * pm + 1) * KP + 8 * ps) = ok1 ? k1 : z;
    *reinterpret_cast<u32x4*>(Ql + (2 * pm) * KP + 8 * ps) = ok0 ? q0 : z;
    *reinterpret_cast<u32x4*>(Ql + (2 * pm + 1) * KP + 8 * ps) = ok1 ? q1 : z;
  };
  auto stage_tv = [&](int par) {
    *reinterpret_cast<u32x4*>(Tp + ti * TP + 8 * tc) = t0;
    *reinterpret_cast<u32x4*>(Tp + PC * TP + ti * TP + 8 * tc) = t1;
    *reinterpret_cast<u32x4*>(Tp + 2 * PC * TP + ti * TP + 8 * tc) = t2;
    // V^T of the chain lane's (row, 4 tokens) into the slots of the first rhs^T
    // plane: the chain lane reads them back and overwrites them with rhs
    uint32_t vz[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vz[q] = tok_ok(tv_c, vi + q) ? v4[q] : 0u;
    *reinterpret_cast<uint2*>(Rp + vr * TP + vi) = make_uint2(vz[0] | (vz[1] << 16), vz[2] | (vz[3] << 16));
    if (st < 64) {
      float* gp = G + 192 * par;
      gp[st] = gv;
      gp[64 + st] = expf(gv);
      gp[128 + st] = tok_ok(tv_c, st) ? bv : 0.f;  // padding: beta = 0
    }
  };
  // K^T of the staged K (tokens 2 pm, 2 pm + 1 of dims [8 ps, +8) per thread)
  auto stage_kt = [&]() {
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(Kl + (2 * pm) * KP + 8 * ps);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(Kl + (2 * pm + 1) * KP + 8 * ps);
    uint32_t* kt = reinterpret_cast<uint32_t*>(KT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of both words
      kt[kt_index(8 * ps + e, 2 * pm) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
    }
  };
  if (NC > 0) {
    load_kq(0);
    load_tv(0);
    stage_kq();
    stage_tv(0);
    load_kq(NC > 1 ? 1 : 0);
    load_tv(NC > 1 ? 1 : 0);
    __syncthreads();
    stage_kt();
    build_m_tile(sw, G);
    if (sw == 2 || sw == 3) build_m_tile(sw + 8, G);
  }
  __syncthreads();

  const int it = sw >> 1, i0 = it * 16 + 4 * lq, nks = (it >> 1) + 1;
  // this sequence's outputs, bounded at its new tokens (a buffered prefix has
  // no outputs here: decode gave them)
  const rsrc_t o_rsrc = make_rsrc(static_cast<char*>(a.o) + tokb * HD * (OUT_BF16 ? 2 : 4),
                                  uint32_t(size_t(Tb - npre) * HD * (OUT_BF16 ? 2 : 4)));
  for (int c = 0; c < NC; ++c) {
    const float* gc = G + 192 * (c & 1);
    // ---- A: output base diag(gamma s) Q S0^T of this wave's (token tile, row tile)
    float os[4];
    {
      f32x4 qacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        qacc = mfma16(lds_bf16x8(Ql + (it * 16 + lr) * KP + kk), lds_bf16x8(Cb + vr * CBP + kk), qacc);
      }
      const float sr = sl[vr];
      const float4 e4 = *reinterpret_cast<const float4*>(gc + 64 + i0);
      const float ge[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) os[q] = ge[q] * (sr * qacc[q]);
    }
    __syncthreads();

    // ---- B: K and Q of this chunk are no longer read.  The loads are
    //      unconditional (the chunk index is clamped), so the in-order load
    //      counter never has to assume the shorter path.
    stage_kq();
    load_kq(c + 2 < NC ? c + 2 : NC - 1);
    __syncthreads();

    // ---- C: O = base + M U; T and the rhs planes were last read in B, and
    //      the other g parity is free
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < nks; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        const bf16x8 m1 = lds_bf16x8(Mp + (it * 16 + lr) * TP + kk);
        const bf16x8 m2 = lds_bf16x8(Mp + PC * TP + (it * 16 + lr) * TP + kk);
        const bf16x8 v1 = lds_bf16x8(Up + vr * TP + kk);
        const bf16x8 v2 = lds_bf16x8(Up + RWS * TP + vr * TP + kk);
        acc = mfma16(m2, v1, acc);
        acc = mfma16(m1, v2, acc);
        acc = mfma16(m1, v1, acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // stores past the sequence (padding tokens) are dropped
        const int tk = c * PC + i0 + q - npre;  // new token of this position (< 0: buffered, no output)
        const uint32_t oi = uint32_t(tk) * HD32 + uint32_t(h * PD + r0 + vr);
        const float ov = os[q] + acc[q];
        if constexpr (OUT_BF16)
          __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_bits(ov)), o_rsrc, tk >= 0 ? oi * 2 : 0xfffffff0u, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), o_rsrc, tk >= 0 ? oi * 4 : 0xfffffff0u, 0, 0);
      }
    }
    stage_tv((c + 1) & 1);
    load_tv(c + 2 < NC ? c + 2 : NC - 1);
    __syncthreads();

    // ---- D: K^T and eight tiles of M of the next chunk (the chain waves 0
    //      and 1 take tiles 8 and 9 beside the requantization)
    if (c + 1 < NC) {
      stage_kt();
      build_m_tile(sw, G + 192 * ((c + 1) & 1));
      if (sw == 2 || sw == 3) build_m_tile(sw + 8, G + 192 * ((c + 1) & 1));
    }
    __syncthreads();
  }
}

// Chunks the workspace holds: B ceil(T / 64) for uniform lengths; for
// variable lengths summing to N new tokens, sum ceil(n / 64) <= floor(N / 64)
// + B, and with a buffered prefix of at most 63 writes per sequence,
// sum ceil((pre + n) / 64) <= floor(N / 64) + 2 B.
static size_t gdn_new_tokens(const PrefillLaunch& L) { return L.varlen ? size_t(L.T) : size_t(L.B) * L.T; }
// d_k = d_v = 64: the head runs as a d = 128 head whose extra key
// dimensions and value rows are zero.  Keys padded with zeros get and erase
// nothing in the extra columns, zero value rows write nothing, and every
// product and row absmax only gains +0 terms, so the padded head carries the
// d = 64 state exactly in its first 64 rows and columns.  gdn_pad_kernel
// widens q, k, v (and the stored state) into the workspace; gdn_unpad_kernel
// copies the outputs and the final state back.
struct PadArgs {
  const uint16_t* x[3];  // q, k, v [rows][64] bf16
  uint16_t* y[3];        // [rows][128] bf16
  int64_t rows;
  const int8_t* c0;      // stored state [bh][64][RB64] (NULL: zero state)
  const float* s0;       // [bh][64]
  int8_t* pc0;           // [bh][128][RB128]
  float* ps0;            // [bh][128]
  int64_t bh;
  int rb64;              // bytes per stored row: 64 (8-bit) or 32 (4-bit)
};

__global__ __launch_bounds__(256) void gdn_pad_kernel(PadArgs a) {
  const int64_t n = a.rows * 3 * 16;  // 16-byte granules of the padded rows
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256) {
    const int64_t row = e / 48;
    const int op = int(e % 48) / 16, g = int(e % 16);
    const uint4 w = g < 8 ? reinterpret_cast<const uint4*>(a.x[op] + row * 64)[g] : make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(a.y[op] + row * PD)[g] = w;
  }
  if (!a.pc0) return;
  const int rb128 = 2 * a.rb64;
  const int64_t ns = a.bh * PD * (rb128 / 16);
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ns; e += int64_t(gridDim.x) * 256) {
    const int64_t r = e / (rb128 / 16);  // padded state row (bh * 128 + row)
    const int g = int(e % (rb128 / 16));
    const int64_t bh = r / PD, rr = r % PD;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (rr < 64 && g < a.rb64 / 16) w = reinterpret_cast<const uint4*>(a.c0 + (bh * 64 + rr) * a.rb64)[g];
    reinterpret_cast<uint4*>(a.pc0 + r * rb128)[g] = w;
    if (g == 0) a.ps0[r] = rr < 64 ? a.s0[bh * 64 + rr] : 0.f;
  }
}

struct UnpadArgs {
  const char* po;  // [rows][128] outputs (eo bytes each)
  char* o;         // [rows][64]
  int64_t rows;
  int eo;
  const int8_t* pc;  // [bh][128][RB128]
  const float* ps;
  int8_t* c;         // [bh][64][RB64]
  float* sc;
  int64_t bh;
  int rb64;
};

__global__ __launch_bounds__(256) void gdn_unpad_kernel(UnpadArgs a) {
  const int gpr = 64 * a.eo / 16;  // 16-byte granules per output row
  const int64_t n = a.rows * gpr;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256) {
    const int64_t row = e / gpr;
    const int g = int(e % gpr);
    reinterpret_cast<uint4*>(a.o + row * 64 * a.eo)[g] = reinterpret_cast<const uint4*>(a.po + row * PD * a.eo)[g];
  }
  const int64_t ns = a.bh * 64 * (a.rb64 / 16);
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ns; e += int64_t(gridDim.x) * 256) {
    const int64_t r = e / (a.rb64 / 16);  // bh * 64 + row
    const int g = int(e % (a.rb64 / 16));
    const int64_t bh = r / 64, rr = r % 64;
    reinterpret_cast<uint4*>(a.c + r * a.rb64)[g] = reinterpret_cast<const uint4*>(a.pc + (bh * PD + rr) * 2 * a.rb64)[g];
    if (g == 0) a.sc[r] = a.ps[bh * PD + rr];
  }
}

// Rotation of q and k (GDNQ_FLAG_WHT): every token row x -> H x / sqrt(128)
// (Sylvester order) in fp32, rounded to bf16 (nearest even): the operand
// precision of the chunk products.  Four lanes per row: five butterfly
// stages inside a lane, the last two across the lane quad through DPP.
// Rows past the end are not written.
struct RotateArgs {
  const uint16_t* x[2];  // q, k [rows][128] bf16
  uint16_t* y[2];        // rotated rows [rows][128] bf16
  int64_t rows;
};

__global__ __launch_bounds__(256) void gdn_rotate_kernel(RotateArgs a) {
  constexpr int LPR = 4, E = PD / LPR;
  const int op = blockIdx.y;
  const int tid = threadIdx.x;
  const int li = tid % LPR;
  const int64_t row = int64_t(blockIdx.x) * (256 / LPR) + tid / LPR;
  const bool valid = row < a.rows;
  float v[E];
  const uint4* src = reinterpret_cast<const uint4*>(a.x[op] + row * PD + li * E);
#pragma unroll
  for (int p = 0; p < E / 8; ++p) {
    const uint4 w = valid ? src[p] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * p + 2 * i] = bf16_lo(ww[i]);
      v[8 * p + 2 * i + 1] = bf16_hi(ww[i]);
    }
  }
  fwht_local<E>(v);
  const bool up1 = (li & 1) != 0, up2 = (li & 2) != 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float o = dpp<DPP_XOR1>(v[i]);
    v[i] = up1 ? (o - v[i]) : (v[i] + o);
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float o = dpp<DPP_XOR2>(v[i]);
    v[i] = up2 ? (o - v[i]) : (v[i] + o);
  }
  if (!valid) return;
  uint4* dst = reinterpret_cast<uint4*>(a.y[op] + row * PD + li * E);
#pragma unroll
  for (int p = 0; p < E / 8; ++p) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32_to_bf16_bits(v[8 * p + 2 * i] * 0.08838834764831845f) |
             (f32_to_bf16_bits(v[8 * p + 2 * i + 1] * 0.08838834764831845f) << 16);
    dst[p] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

static size_t gdn_chunks(const PrefillLaunch& L) {
  if (L.resume) return gdn_new_tokens(L) / PC + 2 * size_t(L.B);
  return L.varlen ? size_t(L.T / PC) + size_t(L.B) : size_t(L.B) * ((L.T + PC - 1) / PC);
}
static size_t gdn_ws_T(const PrefillLaunch& L) { return gdn_chunks(L) * L.H * 3 * PC * PC * 2; }
static size_t gdn_ws_g(const PrefillLaunch& L) { return gdn_chunks(L) * L.H * PC * 4; }
// staged chunk 0 when resuming: k, q, v bf16 [B][64][H][128], alpha, beta fp32 [B][64][H]
static size_t gdn_ws_stage(const PrefillLaunch& L) {
  return L.resume ? size_t(L.B) * PC * L.H * (3 * PD * 2 + 2 * 4) : 0;
}
static bool gdn_mapped(const PrefillLaunch& L) { return L.varlen || L.resume; }
static size_t gdn_ws_map(const PrefillLaunch& L) { return gdn_mapped(L) ? (4 * size_t(L.B) + 2) * 4 : 0; }
// rotated q and k (GDNQ_FLAG_WHT, whole windows only): [2][B*T*H][128] bf16
static size_t gdn_ws_rot(const PrefillLaunch& L) { return L.wht ? 2 * size_t(L.B) * L.T * L.H * PD * 2 : 0; }
constexpr int ORDER_MAXB = 1024;  // sequences ranked by length (more: taken in order)

// Sequence map, one workgroup.  Token offsets tok[i]: with cu, the running
// maximum of cu[i] clamped to [0, T] (so lengths are never negative and
// never reach past the tokens), else i T.  Prefixes pre[i]: fill[i] clamped
// to [0, 63], or 0.  Chunk offsets ch[i]: the sum over the earlier sequences
// of ceil((pre + n) / 64).  A well-formed cu (0 = cu[0] <= ... <= cu[B] = T)
// and fills in [0, 63] pass through unchanged.
struct SeqMapArgs {
  const int32_t* cu;
  const int32_t* fill;
  int32_t* tok;
  int32_t* ch;
  int32_t* pre;
  int32_t* order;  // [B]: sequence of rank r (most chunks first, ties by index)
  int B, T;
};

__global__ __launch_bounds__(1024) void gdn_seqmap_kernel(SeqMapArgs a) {
  __shared__ int32_t sv[1025];
  __shared__ int32_t sc[1024];
  __shared__ int32_t nb[ORDER_MAXB];  // chunks per sequence, for the ranking
  const int t = threadIdx.x;
  auto off = [&](int i) { return a.cu ? min(max(a.cu[i], 0), a.T) : i * a.T; };
  int carry_tok = 0, carry_ch = 0;
  for (int base = 0; base <= a.B; base += 1024) {
    // running maximum of the offsets base .. base + 1024
    const int i = base + t;
    int x = i <= a.B ? off(i) : INT_MAX;
    if (base > 0) x = max(x, carry_tok);
    sv[t] = x;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int y = t >= o ? sv[t - o] : 0;
      __syncthreads();
      sv[t] = max(sv[t], y);
      __syncthreads();
    }
    if (t == 0) sv[1024] = base + 1024 <= a.B ? max(off(base + 1024), sv[1023]) : INT_MAX;
    __syncthreads();
    // positions of sequence i, its chunks, then their exclusive running sum
    const int p = i < a.B && a.fill ? min(max(a.fill[i], 0), PC - 1) : 0;
    const int n = i < a.B ? (p + sv[t + 1] - sv[t] + PC - 1) / PC : 0;
    sc[t] = n;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int y = t >= o ? sc[t - o] : 0;
      __syncthreads();
      sc[t] += y;
      __syncthreads();
    }
    if (i <= a.B) {
      a.tok[i] = sv[t];
      a.ch[i] = carry_ch + sc[t] - n;
    }
    if (i < a.B) a.pre[i] = p;
    if (i < a.B && i < ORDER_MAXB) nb[i] = n;
    carry_tok = sv[1023];
    carry_ch += sc[1023];
    __syncthreads();
  }
  // longest first: rank = sequences with more chunks, or as many and a lower index
  if (a.B <= ORDER_MAXB) {
    for (int i = t; i < a.B; i += 1024) {
      const int n = nb[i];
      int r = 0;
      for (int j = 0; j < a.B; ++j) {
        const int m = nb[j];
        r += (m > n) || (m == n && j < i);
      }
      a.order[r] = i;
    }
  } else {
    for (int i = t; i < a.B; i += 1024) a.order[i] = i;
  }
}

// Chunk 0 of every sequence when resuming, laid out like the tokens: its
// pre buffered writes (fp32 in decode's window buffer, entered at bf16 like
// every prefill token; no query, no output), then its first new tokens, then
// padding (k = q = v = 0, alpha = 1, beta = 0).  One workgroup per
// (sequence, head).
struct StageArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  const float* buf_k;
  const float* buf_v;
  const float* buf_alpha;
  const float* buf_beta;
  uint16_t* sk;
  uint16_t* sq;
  uint16_t* sv;
  float* sa;
  float* sb;
  SeqMap sm;
  int B, H, W;
};

__global__ __launch_bounds__(256) void gdn_stage_kernel(StageArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int pre = a.sm.npre(b), n = a.sm.ntok(b);
  const size_t tok0 = a.sm.tok0(b);
  const size_t HD = size_t(a.H) * PD;
  for (int e = threadIdx.x; e < PC * PD / 2; e += 256) {  // two dims per thread
    const int pos = e / (PD / 2), d = 2 * (e % (PD / 2));
    uint32_t kw = 0u, qw = 0u, vw = 0u;
    if (pos < pre) {
      const size_t src = (size_t(bh) * a.W + pos) * PD + d;
      const float2 kf = *reinterpret_cast<const float2*>(a.buf_k + src);
      const float2 vf = *reinterpret_cast<const float2*>(a.buf_v + src);
      kw = f32_to_bf16_bits(kf.x) | (f32_to_bf16_bits(kf.y) << 16);
      vw = f32_to_bf16_bits(vf.x) | (f32_to_bf16_bits(vf.y) << 16);
    } else if (pos - pre < n) {
      const size_t src = (tok0 + (pos - pre)) * HD + size_t(h) * PD + d;
      kw = *reinterpret_cast<const uint32_t*>(a.k + src);
      qw = *reinterpret_cast<const uint32_t*>(a.q + src);
      vw = *reinterpret_cast<const uint32_t*>(a.v + src);
    }
    const size_t dst = ((size_t(b) * PC + pos) * a.H + h) * PD + d;
    *reinterpret_cast<uint32_t*>(a.sk + dst) = kw;
    *reinterpret_cast<uint32_t*>(a.sq + dst) = qw;
    *reinterpret_cast<uint32_t*>(a.sv + dst) = vw;
  }
  for (int pos = threadIdx.x; pos < PC; pos += 256) {
    float al = 1.f, be = 0.f;
    if (pos < pre) {
      al = a.buf_alpha[size_t(bh) * a.W + pos];
      be = a.buf_beta[size_t(bh) * a.W + pos];
    } else if (pos - pre < n) {
      al = a.alpha[(tok0 + (pos - pre)) * a.H + h];
      be = a.beta[(tok0 + (pos - pre)) * a.H + h];
    }
    a.sa[(size_t(b) * PC + pos) * a.H + h] = al;
    a.sb[(size_t(b) * PC + pos) * a.H + h] = be;
  }
}

// Hand-over to decode: with r = len mod 64 for a sequence of len positions,
// its last r positions' writes go to slots 0 .. r-1 of its window buffer
// (fp32, keys in the state's basis) and its fill becomes r.  Slots that
// already hold a buffered prefix write (when resuming, before any window
// closed) are left as they are.  One workgroup per (sequence, head).
struct HandoffArgs {
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* buf_k;
  float* buf_v;
  float* buf_alpha;
  float* buf_beta;
  int32_t* fill_out;
  SeqMap sm;
  int B, H, W;
};

__global__ __launch_bounds__(256) void gdn_handoff_kernel(HandoffArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int len = a.sm.len(b), pre = a.sm.npre(b);
  const int r = len % PC;
  const int p0 = len - r;  // position of slot 0
  const int s0 = max(pre - p0, 0);  // first slot that takes a new token
  const size_t t0 = a.sm.tok0(b);
  for (int e = threadIdx.x; e < (r - s0) * (PD / 8); e += 256) {  // 8 dims per thread
    const int slot = s0 + e / (PD / 8), d = 8 * (e % (PD / 8));
    const size_t src = ((t0 + (p0 + slot - pre)) * a.H + h) * PD + d;
    const size_t dst = (size_t(bh) * a.W + slot) * PD + d;
    const uint4 kw = *reinterpret_cast<const uint4*>(a.k + src);
    const uint4 vw = *reinterpret_cast<const uint4*>(a.v + src);
    auto widen = [](uint32_t w, float& lo, float& hi) {
      lo = __uint_as_float(w << 16);
      hi = __uint_as_float(w & 0xffff0000u);
    };
    float4 k0, k1, v0, v1;
    widen(kw.x, k0.x, k0.y); widen(kw.y, k0.z, k0.w); widen(kw.z, k1.x, k1.y); widen(kw.w, k1.z, k1.w);
    widen(vw.x, v0.x, v0.y); widen(vw.y, v0.z, v0.w); widen(vw.z, v1.x, v1.y); widen(vw.w, v1.z, v1.w);
    *reinterpret_cast<float4*>(a.buf_k + dst) = k0;
    *reinterpret_cast<float4*>(a.buf_k + dst + 4) = k1;
    *reinterpret_cast<float4*>(a.buf_v + dst) = v0;
    *reinterpret_cast<float4*>(a.buf_v + dst + 4) = v1;
  }
  for (int slot = s0 + threadIdx.x; slot < r; slot += 256) {
    const size_t src = (t0 + (p0 + slot - pre)) * a.H + h;
    a.buf_alpha[size_t(bh) * a.W + slot] = a.alpha[src];
    a.buf_beta[size_t(bh) * a.W + slot] = a.beta[src];
  }
  if (h == 0 && threadIdx.x == 0) a.fill_out[b] = r;
}

static size_t gdn_ws_128(const PrefillLaunch& L) {
  return gdn_ws_T(L) + gdn_ws_g(L) + gdn_ws_stage(L) + gdn_ws_map(L) + gdn_ws_rot(L);
}
// d = 64 through a padded d = 128 head: q, k, v [3][rows][128] bf16, the
// padded stored state and final state ([bh][128][RB128] + [bh][128] each),
// the padded outputs [rows][128]; then the d = 128 workspace
struct PadLayout {
  size_t qkv, c0, s0, o, c, sc, inner, total;
};
static PadLayout gdn_pad_layout(const PrefillLaunch& L) {
  const size_t rows = size_t(L.B) * L.T * L.H, bh = size_t(L.B) * L.H;
  const size_t rb = L.q4 ? PD / 2 : PD, eo = L.out_bf16 ? 2 : 4;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  PadLayout p{};
  p.qkv = 0;
  p.c0 = p.qkv + up(3 * rows * PD * 2);
  p.s0 = p.c0 + up(bh * PD * rb);
  p.o = p.s0 + up(bh * PD * 4);
  p.c = p.o + up(rows * PD * eo);
  p.sc = p.c + up(bh * PD * rb);
  p.inner = p.sc + up(bh * PD * 4);
  PrefillLaunch L2 = L;
  L2.d_k = L2.d_v = PD;
  p.total = p.inner + gdn_ws_128(L2);
  return p;
}

size_t prefill_gdn_workspace_bytes(const PrefillLaunch& L) {
  if (L.d_k == 64) return gdn_pad_layout(L).total;
  return gdn_ws_128(L);
}

static hipError_t launch_prefill_gdn128(const PrefillLaunch& Lin, hipStream_t stream);

hipError_t launch_prefill_gdn(const PrefillLaunch& L, hipStream_t stream) {
  if (L.d_k != 64) return launch_prefill_gdn128(L, stream);
  // d = 64: pad, run the d = 128 kernels on the workspace copies, unpad
  const PadLayout P = gdn_pad_layout(L);
  char* ws = static_cast<char*>(L.workspace);
  const int64_t rows = int64_t(L.B) * L.T * L.H, bh = int64_t(L.B) * L.H;
  const int rb64 = L.q4 ? 32 : 64;
  uint16_t* pq = reinterpret_cast<uint16_t*>(ws + P.qkv);
  PadArgs pa{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v)},
             {pq, pq + rows * PD, pq + 2 * rows * PD}, rows, L.init_codes, L.init_scales,
             L.init_codes ? reinterpret_cast<int8_t*>(ws + P.c0) : nullptr, reinterpret_cast<float*>(ws + P.s0), bh, rb64};
  const int64_t work = rows * 48 > bh * PD * 8 ? rows * 48 : bh * PD * 8;
  const unsigned grid = unsigned(work / 256 + 1 < 4096 ? work / 256 + 1 : 4096);
  hipLaunchKernelGGL(gdn_pad_kernel, dim3(grid), dim3(256), 0, stream, pa);
  if (hipError_t e = hipGetLastError()) return e;
  PrefillLaunch L2 = L;
  L2.d_k = L2.d_v = PD;
  L2.q = pa.y[0];
  L2.k = pa.y[1];
  L2.v = pa.y[2];
  L2.init_codes = pa.pc0;
  L2.init_scales = L.init_codes ? pa.ps0 : nullptr;
  L2.o = ws + P.o;
  L2.codes = reinterpret_cast<int8_t*>(ws + P.c);
  L2.scales = reinterpret_cast<float*>(ws + P.sc);
  L2.workspace = ws + P.inner;
  if (hipError_t e = launch_prefill_gdn128(L2, stream)) return e;
  UnpadArgs ua{ws + P.o, static_cast<char*>(L.o), rows, L.out_bf16 ? 2 : 4, L2.codes, L2.scales, L.codes, L.scales,
               bh, rb64};
  hipLaunchKernelGGL(gdn_unpad_kernel, dim3(grid), dim3(256), 0, stream, ua);
  return hipGetLastError();
}

static hipError_t launch_prefill_gdn128(const PrefillLaunch& Lin, hipStream_t stream) {
  PrefillLaunch L = Lin;
  char* ws = static_cast<char*>(L.workspace);
  if (L.wht && L.B > 0 && L.T > 0) {  // rotate q and k once; the chunk kernels read the rotated rows
    uint16_t* rq = reinterpret_cast<uint16_t*>(ws + gdn_ws_T(L) + gdn_ws_g(L) + gdn_ws_stage(L) + gdn_ws_map(L));
    const int64_t rows = int64_t(L.B) * L.T * L.H;
    uint16_t* rk = rq + rows * PD;
    RotateArgs ra{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k)}, {rq, rk}, rows};
    hipLaunchKernelGGL(gdn_rotate_kernel, dim3(unsigned((rows + 63) / 64), 2), dim3(256), 0, stream, ra);
    if (hipError_t e = hipGetLastError()) return e;
    L.q = rq;
    L.k = rk;
  }
  __bf16* T_ws = reinterpret_cast<__bf16*>(ws);
  float* g_ws = reinterpret_cast<float*>(ws + gdn_ws_T(L));
  SeqMap sm{};
  sm.T = L.T;
  if (gdn_mapped(L)) {
    char* st = ws + gdn_ws_T(L) + gdn_ws_g(L);
    int32_t* tok = reinterpret_cast<int32_t*>(st + gdn_ws_stage(L));
    int32_t* ch = tok + (L.B + 1);
    int32_t* pre = ch + (L.B + 1);
    int32_t* order = pre + L.B;
    SeqMapArgs m{L.cu_seqlens, L.resume ? L.fill_in : nullptr, tok, ch, pre, order, L.B, L.T};
    hipLaunchKernelGGL(gdn_seqmap_kernel, dim3(1), dim3(1024), 0, stream, m);
    if (hipError_t e = hipGetLastError()) return e;
    sm.tok = tok;
    sm.ch = ch;
    sm.order = order;  // read by the state kernel only
    if (L.resume) {
      const size_t nstage = size_t(L.B) * PC * L.H;
      uint16_t* sk = reinterpret_cast<uint16_t*>(st);
      uint16_t* sq = sk + nstage * PD;
      uint16_t* sv = sq + nstage * PD;
      float* sa = reinterpret_cast<float*>(sv + nstage * PD);
      float* sb = sa + nstage;
      StageArgs g{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k),
                  static_cast<const uint16_t*>(L.v), L.alpha, L.beta, L.buf_k, L.buf_v, L.buf_alpha,
                  L.buf_beta, sk, sq, sv, sa, sb, sm, L.B, L.H, L.W};
      g.sm.pre = pre;  // the staging kernel reads the prefixes, not yet the staged copy
      hipLaunchKernelGGL(gdn_stage_kernel, dim3(unsigned(L.B) * L.H), dim3(256), 0, stream, g);
      if (hipError_t e = hipGetLastError()) return e;
      sm.pre = pre;
      sm.sk = sk; sm.sq = sq; sm.sv = sv; sm.sa = sa; sm.sb = sb;
    }
  }
  const size_t nch = gdn_chunks(L);
  if (nch > 0) {
    const size_t total = nch * L.H;
    PrepArgs p{static_cast<const uint16_t*>(L.k), L.alpha, L.beta, T_ws, g_ws, sm, L.B, L.H, int(total)};
    // four resident workgroups per CU (LDS): each loops over chunk-heads
    const unsigned grid = unsigned(total < PREP_GRID ? total : PREP_GRID);
    hipLaunchKernelGGL(gdn_prep_kernel, dim3(grid), dim3(256), 0, stream, p);
    if (hipError_t e = hipGetLastError()) return e;
  }
  StateArgs s{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k),
              static_cast<const uint16_t*>(L.v), L.beta, T_ws, g_ws, L.init_codes, L.init_scales,
              L.o, L.codes, L.scales, sm, L.B, L.H};
  const unsigned grid = unsigned(L.B) * L.H * (PD / RWS);
  auto kern = L.q4 ? (L.out_bf16 ? &gdn_state_kernel<true, 4> : &gdn_state_kernel<false, 4>)
                   : (L.out_bf16 ? &gdn_state_kernel<true, 8> : &gdn_state_kernel<false, 8>);
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, STATE_LDS))
    return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(SNT), STATE_LDS, stream, s);
  if (hipError_t e = hipGetLastError()) return e;
  if (L.handoff && L.B > 0) {
    HandoffArgs h{static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v), L.alpha, L.beta,
                  L.buf_k, L.buf_v, L.buf_alpha, L.buf_beta, L.fill_out, sm, L.B, L.H, L.W};
    hipLaunchKernelGGL(gdn_handoff_kernel, dim3(unsigned(L.B) * L.H), dim3(256), 0, stream, h);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdnq
