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
//            blocks on fp32 MFMA); T's ten lower 16x16 tiles (as three bf16
//            parts) and g go to the workspace.
//   state -- one workgroup per (sequence, head, block of 32 rows): rows of
//            the state evolve independently, so each workgroup carries its
//            rows through all chunks.  Two chain waves hold 16 rows each
//            entirely in registers (codes, rhs, U, U o d) and run a chunk's
//            recurrence without waiting on any other wave; side waves form
//            the output one chunk behind, staging waves load and stage the
//            next chunk; one barrier per chunk.  Every product runs on bf16
//            MFMA: K S0^T and Q S0^T take the codes exactly; T (rhs),
//            K^T (U o d) and M U split their fp32 operands into two or three
//            bf16 parts, which keeps fp32-level accuracy.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "mfma.h"

namespace gdnq {

constexpr int PC = 64;    // chunk = window
constexpr int PD = 128;   // d_k = d_v
constexpr int RWS = 32;   // state rows per state-pass workgroup
constexpr int TT = 10;    // lower 16x16 tiles of a 64x64 matrix (T is kept as these)

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
// A and T are kept as their ten lower 16x16 tiles (the upper ones are zero):
// tile (ti, tj), ti >= tj, is tile ti (ti + 1) / 2 + tj, rows of AQ / TQ
// floats (17: the level products read A down a column without bank
// conflicts; 20: T's rows stay 16-byte aligned and a column read is
// conflict-free)
constexpr int AQ = 17, TQ = 20;
constexpr int PREP_GRID = 5 * 256;  // prep workgroups: five per CU
constexpr int PREP_T = (TT * 16 * TQ + 3 * 256) * 4;  // T tiles, then the level products
constexpr int PREP_KT = PC * KP * 2 > PREP_T ? PC * KP * 2 : PREP_T;
__device__ __forceinline__ int ltile(int ti, int tj) { return ti * (ti + 1) / 2 + tj; }  // tj <= ti

struct PrepArgs {
  const uint16_t* k;
  const float* alpha;
  const float* beta;
  __bf16* T_ws;  // [chunks*H][3][10][16][16]: T's lower tiles as hi/mid/lo bf16 parts
  float* g_ws;  // [chunks*H][64]
  SeqMap sm;
  int B, H;
  int total;  // chunk-heads the grid covers (an upper bound when mapped)
};

__global__ __launch_bounds__(256, 5) void gdn_prep_kernel(PrepArgs a) {
  // K is only needed for K K^T; T and the level products reuse its space
  __shared__ __attribute__((aligned(16))) unsigned char kt_raw[PREP_KT];
  __shared__ float Al[TT * 16 * AQ];
  __shared__ float gl[PC], bl[PC];
  __bf16* Kl = reinterpret_cast<__bf16*>(kt_raw);
  float* Tl = reinterpret_cast<float*>(kt_raw);
  float* Pl = Tl + TT * 16 * TQ;
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
      // row offsets by 24-bit products: a 32-bit product formed with a 64-bit
      // multiply-add reads an unrelated register as its high half, and a load
      // of the next chunk-head still in flight there would be waited for
      const __bf16* ki = Kl + __umul24(uint32_t(it * 16 + lr), uint32_t(KP));
      const __bf16* kj = Kl + __umul24(uint32_t(jt * 16 + lr), uint32_t(KP));
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * lq;
        acc = mfma16(lds_bf16x8(ki + kk), lds_bf16x8(kj + kk), acc);
      }
      const int j = jt * 16 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = it * 16 + 4 * lq + q;
        // e^(g_i - g_j) <= 1 by the hardware exp2 (the argument is <= 0; a
        // result below fp32's normal range is 0)
        av[n][q] = (j < i) ? bl[i] * __builtin_amdgcn_exp2f((gl[i] - gl[j]) * 1.4426950408889634f) * acc[q] : 0.f;
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
      for (int q = 0; q < 4; ++q) Al[(tt * 16 + 4 * lq + q) * AQ + lr] = av[n][q];
    }
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
      for (int j = 0; j < r; ++j) s -= Al[(ltile(bb, bb) * 16 + r) * AQ + j] * t[j];
      t[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tl[(ltile(bb, bb) * 16 + r) * TQ + cc] = t[r];
  }
  __syncthreads();

  // off-diagonal blocks (fp32 MFMA), wave j the blocks of column j in turn,
  // i = j + 1 .. 3:  P = sum_{k=j}^{i-1} A_ik T_kj,  T_ij = -T_ii P.  A block
  // needs only its own column's blocks above it and the diagonal, so the
  // waves exchange nothing; within a wave the LDS round trips (P, then the
  // new block) are ordered by wavefront fences.
  if (wave < 3) {
    const int j = wave;
    for (int i = j + 1; i < 4; ++i) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = j; kb < i; ++kb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma4(Al[(ltile(i, kb) * 16 + lr) * AQ + 4 * kk + lq], Tl[(ltile(kb, j) * 16 + 4 * kk + lq) * TQ + lr], acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) Pl[wave * 256 + (4 * lq + q) * 16 + lr] = acc[q];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        t = mfma4(Tl[(ltile(i, i) * 16 + lr) * TQ + 4 * kk + lq], Pl[wave * 256 + (4 * kk + lq) * 16 + lr], t);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // P is read before the next block overwrites it
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) Tl[(ltile(i, j) * 16 + 4 * lq + q) * TQ + lr] = -t[q];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  {  // T's ten lower 16x16 tiles as three bf16 parts [part][tile][16][16]:
     // thread -> row tid / 4, columns [(tid % 4) * 16, +16), tiles on or below the diagonal
    const int i = tid >> 2, c0 = (tid & 3) * 16;
    const int ti = i >> 4, tj = c0 >> 4;
    const int tl = tj <= ti ? ltile(ti, tj) : 0;  // tiles above the diagonal are not stored (nor read)
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 t4 = *reinterpret_cast<const float4*>(Tl + (tl * 16 + (i & 15)) * TQ + e);
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
    if (tj <= ti) {
      __bf16* dst = a.T_ws + size_t(idx) * 3 * TT * 256 + (ti * (ti + 1) / 2 + tj) * 256 + (i & 15) * 16;
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        *reinterpret_cast<bf16x8*>(dst + pl * TT * 256) = p[pl][0];
        *reinterpret_cast<bf16x8*>(dst + pl * TT * 256 + 8) = p[pl][1];
      }
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
  int cpw;  // chunks per window (the state is requantized after every cpw-th); 0: never
  float* state_f32;  // the final fp32 state (never requantized), or NULL
};

constexpr int SNT = 512;  // state-pass threads: 2 chain, 4 side and 2 staging waves
constexpr int VTP = 72;   // bf16 pitch of the V^T rows

// LDS carve (bytes); [2] = by chunk parity
constexpr int L_K = 0;                               // K [2][64][KP] bf16
constexpr int L_Q = L_K + 2 * PC * KP * 2;           // Q [64][KP] bf16 (restaged in place)
constexpr int L_KT = L_Q + PC * KP * 2;              // K^T [2][128][64] bf16, 16-byte granules xor-swizzled
constexpr int L_T = L_KT + 2 * PD * PC * 2;          // T [2][3 parts][10 tiles][16][16] bf16
constexpr int L_V = L_T + 2 * 3 * TT * 256 * 2;      // V^T [2][32][VTP] bf16
constexpr int L_U = L_V + 2 * RWS * VTP * 2;         // U [2][2 parts][2 waves][2 steps][64 lanes] bf16x8
constexpr int L_C = L_U + 2 * 2 * 2 * 2 * 64 * 16;   // codes [2][2 waves][4 steps][64 lanes] bf16x8
constexpr int L_F = L_C + 2 * 2 * 4 * 64 * 16;       // g, exp(g), beta, exp(g_C - g) [2][4][64] fp32
constexpr int L_S = L_F + 2 * 4 * PC * 4;            // row scales [2][32] fp32
constexpr int STATE_LDS = L_S + 2 * RWS * 4;
static_assert(STATE_LDS <= 160 * 1024, "state-pass LDS");

__device__ __forceinline__ int kt_index(int d, int j) {  // bf16 index of K^T[d][j]
  return d * PC + ((((j >> 3) ^ (d >> 3)) & 7) << 3) + (j & 7);
}

__device__ __forceinline__ int tile_index(int it, int jt) { return it * (it + 1) / 2 + jt; }  // jt <= it

__device__ __forceinline__ bf16x4 lds4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

__device__ __forceinline__ bf16x8 cat8(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A 32-wide k step of a 16x16x32 product takes its operands in the order
//   slot 4h + q of lane group g  <->  index (2 ks + h) 16 + 4 g + q,
// the order in which a 16x16 output tile holds four consecutive rows per lane
// group.  Output tiles therefore feed the next product's B operand straight
// from registers, and A operands are read from LDS as two 8-byte halves.
//
// Per workgroup (sequence, head, 32 state rows), eight waves:
// (Waves are placed on the four SIMDs round robin: each chain wave shares its
// SIMD with a staging wave, the lightest role.)
//   chain waves 0, 1 -- 16 rows each, all in registers: the codes and scale
//     of S0, then per chunk X = K codes^T, rhs = beta (v - gamma s X),
//     U = T rhs, S_C^T = gamma_C S0^T + K^T (U o d) and the requantization.
//   side waves 2, 3, 6, 7 -- token tile it = 0, 1, 2, 3: M = L o Q K^T for the tiles
//     (it, <= it) and the output base gamma s Q S0^T, kept in registers, and
//     a chunk later O = base + M U.  Each restages its own 16 rows of Q.
//   staging waves 4, 5 -- K, K^T, T, V^T and the per-token scalars of the
//     next chunk into the other buffer; loads two chunks ahead.
// One barrier per chunk.  In chunk c the chain reads buffer c & 1 and writes
// U_c and the codes of S0_{c+1}; the side waves read U_{c-1} and the codes
// of S0_c; staging fills buffer (c + 1) & 1.
// QB: the state's code width, 8 (int8) or 4 (packed 4-bit, scale absmax / 7)
// CARRY: windows span several chunks (or the state is never requantized).
// Between window ends the chain keeps S0 in fp32 (values in cf, s = 1) and
// takes K S0^T in three bf16 parts; the side waves get S0 as two int8 levels,
// row ~= s1 (c1 + c2 / 254) with s1 = max|row| / 127 (within 1.6e-5 of the
// row's absmax: the output base only), exact where S0 is a requantized state.
template <bool OUT_BF16, int QB, bool CARRY>
__global__ __launch_bounds__(SNT, 1) void gdn_state_kernel(StateArgs a) {
  constexpr int QMAX = QB == 8 ? 127 : 7;
  constexpr int RB = PD * QB / 8;  // bytes per stored row
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __bf16* const Kl = reinterpret_cast<__bf16*>(lds + L_K);
  __bf16* const Ql = reinterpret_cast<__bf16*>(lds + L_Q);
  __bf16* const KTl = reinterpret_cast<__bf16*>(lds + L_KT);
  __bf16* const Tl = reinterpret_cast<__bf16*>(lds + L_T);
  __bf16* const Vl = reinterpret_cast<__bf16*>(lds + L_V);
  bf16x8* const Ul = reinterpret_cast<bf16x8*>(lds + L_U);
  bf16x8* const Cl = reinterpret_cast<bf16x8*>(lds + L_C);
  float* const Fl = reinterpret_cast<float*>(lds + L_F);
  float* const Sl = reinterpret_cast<float*>(lds + L_S);
  auto u_at = [&](int par, int part, int w, int ks) { return Ul + (((par * 2 + part) * 2 + w) * 2 + ks) * 64; };
  auto c_at = [&](int par, int w, int ks) { return Cl + ((par * 2 + w) * 4 + ks) * 64; };

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
  const int bs = a.sm.order && (nblk & 31) == 0 ? a.sm.order[cr / a.H] : chain / a.H;
  const int h = cr % a.H;
  const int r0 = rb * RWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, g4 = lane >> 4;
  const int Tb = a.sm.len(bs);  // this sequence's positions (buffered prefix and new tokens)
  const int NC = (Tb + PC - 1) / PC;
  const bool partial_last = (Tb % PC) != 0;  // the last chunk holds fewer than 64 tokens
  const size_t HD = size_t(a.H) * PD;
  const uint32_t HD32 = uint32_t(HD);
  const size_t state_row0 = (size_t(bs) * a.H + h) * PD + r0;
  const size_t tokb = a.sm.tok0(bs);
  // where chunk c's positions are read (the sequence map is read once, here)
  const int npre = a.sm.npre(bs);
  const bool stg0 = a.sm.pre != nullptr;  // chunk 0 is read from the staged copy
  const size_t row_c0 = stg0 ? size_t(bs) * PC : tokb;
  const size_t row_t = tokb - size_t(npre);  // chunk c >= 1 starts at row row_t + 64 c (wraps back for c >= 1)
  auto chunk_row = [&](int c) { return c == 0 ? row_c0 : row_t + size_t(c) * PC; };
  auto tok_ok = [&](int c, int i) { return c * PC + i < Tb; };
  auto in_row = [&](int c, int i) {  // in-chunk row a load reads, clamped into the sequence
    const int lim = Tb - 1 - c * PC;
    return uint32_t(i < lim ? i : lim);
  };
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  if (wave < 2) {
    // ================================================================ chain waves
    const int rl = wave * 16 + lr;  // this lane's row of the block
    const size_t grow = state_row0 + rl;
    float cf[8][4];  // S0 in units of s: dims dt 16 + 4 g4 + q (codes, or fp32 values with s = 1)
    float s = 0.f;
    if (a.init_codes) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d0 = dt * 16 + 4 * g4;
        uint32_t w;
        if constexpr (QB == 8) w = *reinterpret_cast<const uint32_t*>(a.init_codes + grow * RB + d0);
        else w = *reinterpret_cast<const uint16_t*>(a.init_codes + grow * RB + d0 / 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) cf[dt][q] = code_at<QB>(w, q);
      }
      s = a.init_scales[grow];
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) cf[dt][q] = 0.f;
    }
    bf16x8 cb[4];  // the codes as B operands of X, one per 32-dim step
    auto pack_codes = [&]() {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) cb[ks][e] = (__bf16)cf[2 * ks + (e >> 2)][e & 3];
    };
    auto publish = [&](int par) {  // S0 for the side waves' output base
      if constexpr (!CARRY) {  // the codes (exact in bf16) and the row scale
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) c_at(par, wave, ks)[lane] = cb[ks];
        if (g4 == 0) Sl[par * RWS + rl] = s;
      } else {  // two int8 levels c1, c2 (bytes 0-7, 8-15 of the slot) and s1
        float am = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) am = fmaxf(am, fabsf(cf[dt][q]));
        am = xor32_max(xor16_max(am));  // the row's other three lane groups
        const float inv = am > 0.f ? 127.f / am : 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          uint32_t w[4];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            int c1[4], c2[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float t = cf[2 * ks + hh][q] * inv, r = rintf(t);
              c1[q] = int(r);
              c2[q] = int(rintf((t - r) * 254.f));
            }
            w[hh] = pack4_i8(c1[0], c1[1], c1[2], c1[3]);
            w[2 + hh] = pack4_i8(c2[0], c2[1], c2[2], c2[3]);
          }
          const u32x4 wv = {w[0], w[1], w[2], w[3]};
          *reinterpret_cast<u32x4*>(c_at(par, wave, ks) + lane) = wv;
        }
        if (g4 == 0) Sl[par * RWS + rl] = s * am * (1.f / 127.f);
      }
    };
    if constexpr (!CARRY) pack_codes();
    publish(0);
    // CARRY: chunks since the window began (0: S0 is the stored codes, or zero;
    // never requantizing, only chunk 0)
    int wc = 0;
    __syncthreads();  // chunk 0 staged

    for (int c = 0; c < NC; ++c) {
      const int par = c & 1;
      const __bf16* K = Kl + par * PC * KP;
      const __bf16* KT = KTl + par * PD * PC;
      const __bf16* T = Tl + par * 3 * TT * 256;
      const __bf16* V = Vl + par * RWS * VTP;
      const float* F = Fl + par * 4 * PC;
      // The A operands of X (K) and of U (T) are read up front, so the
      // products issue back to back instead of each waiting for its read.
      bf16x8 ka[4][4];  // K rows of tile jt, step ks
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const __bf16* kr = K + (jt * 16 + lr) * KP + ks * 32 + 4 * g4;
          ka[jt][ks] = cat8(lds4(kr), lds4(kr + 16));
        }
      bf16x8 ta[6][3];  // T parts for (it, ks) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int ks = 0; ks <= (it >> 1); ++ks) {
          const int n = it == 0 ? 0 : it == 1 ? 1 : it == 2 ? 2 + ks : 4 + ks;
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            const __bf16* tp = T + p * TT * 256 + lr * 16 + 4 * g4;
            const bf16x4 lo = lds4(tp + tile_index(it, 2 * ks) * 256);
            bf16x4 hi = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
            if (2 * ks + 1 <= it) hi = lds4(tp + tile_index(it, 2 * ks + 1) * 256);
            ta[n][p] = cat8(lo, hi);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      // ---- X = K S0^T (in units of s): tile jt holds tokens jt 16 + 4 g4 + q of row rl
      f32x4 x[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) x[jt] = {0.f, 0.f, 0.f, 0.f};
      if (CARRY && wc != 0) {  // fp32 S0 inside a window: three bf16 parts (exact)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          float xs[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[e] = cf[2 * ks + (e >> 2)][e & 3];
          bf16x8 ph, pm, pl;
          split3t(xs, ph, pm, pl);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) x[jt] = mfma16(ka[jt][ks], pl, x[jt]);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) x[jt] = mfma16(ka[jt][ks], pm, x[jt]);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) x[jt] = mfma16(ka[jt][ks], ph, x[jt]);
        }
      } else if constexpr (CARRY) {  // a window's first chunk: S0 is codes (or zero), exact in bf16
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 cw;
#pragma unroll
          for (int e = 0; e < 8; ++e) cw[e] = (__bf16)cf[2 * ks + (e >> 2)][e & 3];
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) x[jt] = mfma16(ka[jt][ks], cw, x[jt]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) x[jt] = mfma16(ka[jt][ks], cb[ks], x[jt]);
      }
      // ---- rhs = beta (v - gamma s X) in three bf16 parts
      bf16x8 rp[3][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float rh[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int jt = 2 * ks + hh, i0 = jt * 16 + 4 * g4;
          const float4 ga = *reinterpret_cast<const float4*>(F + PC + i0);
          const float4 be = *reinterpret_cast<const float4*>(F + 2 * PC + i0);
          const uint2 vw = *reinterpret_cast<const uint2*>(V + rl * VTP + i0);
          const float vv[4] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y)};
          const float gg[4] = {ga.x, ga.y, ga.z, ga.w}, bt[4] = {be.x, be.y, be.z, be.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) rh[4 * hh + q] = bt[q] * (vv[q] - gg[q] * (s * x[jt][q]));
        }
        split3t(rh, rp[0][ks], rp[1][ks], rp[2][ks]);
      }
      // ---- U = T rhs (T unit lower triangular, three parts; six split products)
      f32x4 u[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ub = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks <= (it >> 1); ++ks) {
          const bf16x8* t = ta[it == 0 ? 0 : it == 1 ? 1 : it == 2 ? 2 + ks : 4 + ks];
          ua = mfma16(t[1], rp[1][ks], ua);
          ub = mfma16(t[2], rp[0][ks], ub);
          ua = mfma16(t[0], rp[2][ks], ua);
          ub = mfma16(t[1], rp[0][ks], ub);
          ua = mfma16(t[0], rp[1][ks], ua);
          ub = mfma16(t[0], rp[0][ks], ub);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) u[it][q] = ua[q] + ub[q];
      }
      // the update's A operands (K^T), read while U is formed
      bf16x8 kta[8][2];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int d = dt * 16 + lr, j = ks * 32 + 4 * g4;
          kta[dt][ks] = cat8(lds4(KT + kt_index(d, j)), lds4(KT + kt_index(d, j + 16)));
        }
      // ---- U (two parts) for the side waves; U o d (three parts) for the update
      bf16x8 dp[3][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float uu[8], ud[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4 d4 = *reinterpret_cast<const float4*>(F + 3 * PC + (2 * ks + hh) * 16 + 4 * g4);
          const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uu[4 * hh + q] = u[2 * ks + hh][q];
            ud[4 * hh + q] = u[2 * ks + hh][q] * dd[q];
          }
        }
        bf16x8 u1, u2;
        split2t(uu, u1, u2);
        u_at(par, 0, wave, ks)[lane] = u1;
        u_at(par, 1, wave, ks)[lane] = u2;
        split3t(ud, dp[0][ks], dp[1][ks], dp[2][ks]);
      }
      // ---- S_C^T = gamma_C S0^T + K^T (U o d), then requantize the row at a
      //      window end (not for a partial last chunk: its window stays open
      //      and the stored state stays at the last boundary)
      if (!(partial_last && c == NC - 1)) {
        const float gs = F[PC + PC - 1] * s;
        float sn[32];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 ak = kta[dt][ks];
            acc = mfma16(ak, dp[2][ks], acc);
            acc = mfma16(ak, dp[1][ks], acc);
            acc = mfma16(ak, dp[0][ks], acc);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) sn[4 * dt + q] = gs * cf[dt][q] + acc[q];
        }
        if (CARRY) wc = (a.cpw > 0 && wc + 1 == a.cpw) ? 0 : wc + 1;  // 0: chunk c + 1 starts a window
        if (!CARRY || wc == 0) {
          float m4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial maxima
#pragma unroll
          for (int e = 0; e < 32; ++e) m4[e & 3] = fmaxf(m4[e & 3], fabsf(sn[e]));
          // the row's other three lane groups
          const float amax = xor32_max(xor16_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))));
          float cn[32];
          s = codec_row<32, QMAX>(sn, amax, cn);
#pragma unroll
          for (int e = 0; e < 32; ++e) cf[e >> 2][e & 3] = cn[e];
        } else {  // inside a window: the state stays fp32
#pragma unroll
          for (int e = 0; e < 32; ++e) cf[e >> 2][e & 3] = sn[e];
          s = 1.f;
        }
        if constexpr (!CARRY) pack_codes();
        if (c + 1 < NC) publish(par ^ 1);
      }
      __syncthreads();
    }
    if (CARRY && a.state_f32) {  // never requantized: the fp32 rows
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(a.state_f32 + grow * PD + dt * 16 + 4 * g4) =
            make_float4(cf[dt][0] * s, cf[dt][1] * s, cf[dt][2] * s, cf[dt][3] * s);
      return;
    }
    // final rows (codes back to int8, or packed 4-bit)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d0 = dt * 16 + 4 * g4;
      const int c0 = int(cf[dt][0]), c1 = int(cf[dt][1]), c2 = int(cf[dt][2]), c3 = int(cf[dt][3]);
      if constexpr (QB == 8)
        *reinterpret_cast<uint32_t*>(a.codes + grow * RB + d0) = pack4_i8(c0, c1, c2, c3);
      else
        *reinterpret_cast<uint16_t*>(a.codes + grow * RB + d0 / 2) =
            uint16_t((c0 & 0xf) | ((c1 & 0xf) << 4) | ((c2 & 0xf) << 8) | ((c3 & 0xf) << 12));
    }
    if (g4 == 0) a.scales[grow] = s;
    return;
  }

  if (wave != 4 && wave != 5) {
    // ================================================================ side waves
    const int it = wave < 4 ? wave - 2 : wave - 4;  // token tile
    // Q rows it 16 + qrow, 64-byte segment qseg: four 16-byte loads per lane
    const int qrow = lane >> 2, qseg = lane & 3;
    const uint16_t* const q_c0 = stg0 ? a.sm.sq : a.q;
    u32x4 qv[4];
    int q_c = 0;  // the chunk qv holds
    auto load_q = [&](int c) {
      q_c = c;
      const uint16_t* qb = (c == 0 ? q_c0 : a.q) + chunk_row(c) * HD + size_t(h) * PD + qseg * 32;
      const uint32_t o = in_row(c, it * 16 + qrow) * HD32;
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[e] = *reinterpret_cast<const u32x4*>(qb + o + 8 * e);
    };
    auto stage_q = [&]() {
      const bool ok = tok_ok(q_c, it * 16 + qrow);
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(Ql + (it * 16 + qrow) * KP + qseg * 32 + 8 * e) = ok ? qv[e] : z4;
    };
    if (NC > 0) {
      load_q(0);
      stage_q();
      load_q(NC > 1 ? 1 : 0);
    }
    __syncthreads();

    bf16x8 mA[2][2];  // M (tiles (it, 2 ks), (it, 2 ks + 1)) as A operands, hi and lo parts
    f32x4 os[2];      // output base of the two row tiles
    // this sequence's outputs, bounded at its new tokens (a buffered prefix has
    // no outputs here: decode gave them)
    const rsrc_t o_rsrc = make_rsrc(static_cast<char*>(a.o) + tokb * HD * (OUT_BF16 ? 2 : 4),
                                    uint32_t(size_t(Tb - npre) * HD * (OUT_BF16 ? 2 : 4)));
    auto output = [&](int c) {  // O of chunk c = base + M U
      const int par = c & 1;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks <= (it >> 1)) {  // the steps that reach the diagonal of tile it
            const bf16x8 u1 = u_at(par, 0, rt, ks)[lane], u2 = u_at(par, 1, rt, ks)[lane];
            acc = mfma16(mA[ks][1], u1, acc);
            acc = mfma16(mA[ks][0], u2, acc);
            acc = mfma16(mA[ks][0], u1, acc);
          }
        }
        // a 4x4 transpose inside each quad of lanes (two DPP butterfly
        // stages): lane (tokens 4 g4 .. +4, row lr) -> (token 4 g4 + lane % 4,
        // rows lr - lane % 4 .. +4), one vector store per lane.  Stores past
        // the sequence (padding) and of buffered positions are dropped.
        float ov[4] = {os[rt][0] + acc[0], os[rt][1] + acc[1], os[rt][2] + acc[2], os[rt][3] + acc[3]};
        const bool x1 = lane & 1, x2 = lane & 2;
#pragma unroll
        for (int p = 0; p < 4; p += 2) {  // slot bit 0 <-> lane bit 0
          const float w = dpp<DPP_XOR1>(x1 ? ov[p] : ov[p + 1]);
          if (x1) ov[p] = w;
          else ov[p + 1] = w;
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {  // slot bit 1 <-> lane bit 1
          const float w = dpp<DPP_XOR2>(x2 ? ov[p] : ov[p + 2]);
          if (x2) ov[p] = w;
          else ov[p + 2] = w;
        }
        const int tk = c * PC + it * 16 + 4 * g4 + (lane & 3) - npre;  // new token (< 0: buffered)
        const uint32_t oi = uint32_t(tk) * HD32 + uint32_t(h * PD + r0 + rt * 16 + 4 * (lr >> 2));
        if constexpr (OUT_BF16) {
          const u32x2 w = {f32_to_bf16_bits(ov[0]) | (f32_to_bf16_bits(ov[1]) << 16),
                           f32_to_bf16_bits(ov[2]) | (f32_to_bf16_bits(ov[3]) << 16)};
          __builtin_amdgcn_raw_buffer_store_b64(w, o_rsrc, tk >= 0 ? oi * 2 : 0xffffffe0u, 0, 0);
        } else {
          const u32x4 w = {__float_as_uint(ov[0]), __float_as_uint(ov[1]), __float_as_uint(ov[2]),
                           __float_as_uint(ov[3])};
          __builtin_amdgcn_raw_buffer_store_b128(w, o_rsrc, tk >= 0 ? oi * 4 : 0xffffffe0u, 0, 0);
        }
      }
    };
    for (int c = 0; c < NC; ++c) {
      const int par = c & 1;
      const __bf16* K = Kl + par * PC * KP;
      const float* F = Fl + par * 4 * PC;
      if (c > 0) output(c - 1);
      // ---- M = L o Q K^T for tiles (it, jt <= it): the tile D[j][i] = k_j . q_i
      //      holds tokens j = jt 16 + 4 g4 + q for query i = it 16 + lr
      {
        const int i = it * 16 + lr;
        const float gi = F[i];
        float m[4][4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) m[jt][q] = 0.f;
          if (jt <= it) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const int kk = ks * 32 + 8 * g4;
              acc = mfma16(lds_bf16x8(K + (jt * 16 + lr) * KP + kk), lds_bf16x8(Ql + i * KP + kk), acc);
            }
            const float4 g4v = *reinterpret_cast<const float4*>(F + jt * 16 + 4 * g4);
            const float gj[4] = {g4v.x, g4v.y, g4v.z, g4v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int j = jt * 16 + 4 * g4 + q;
              m[jt][q] = (j <= i) ? exp_out(gi - gj[q]) * acc[q] : 0.f;
            }
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
      // ---- output base gamma_i s_r Q S0^T for the two row tiles
      {
        const float4 ga = *reinterpret_cast<const float4*>(F + PC + it * 16 + 4 * g4);
        const float ge[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if constexpr (CARRY) {  // the two int8 levels: s1 (Q c1^T + Q c2^T / 254)
            f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const __bf16* qr = Ql + (it * 16 + lr) * KP + ks * 32 + 4 * g4;
              const bf16x8 qa = cat8(lds4(qr), lds4(qr + 16));
              const u32x4 w = *reinterpret_cast<const u32x4*>(c_at(par, rt, ks) + lane);
              acc = mfma16(qa, i8x8_to_bf16(make_uint2(w[0], w[1])), acc);
              acc2 = mfma16(qa, i8x8_to_bf16(make_uint2(w[2], w[3])), acc2);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += acc2[q] * (1.f / 254.f);
          } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const __bf16* qr = Ql + (it * 16 + lr) * KP + ks * 32 + 4 * g4;
              acc = mfma16(cat8(lds4(qr), lds4(qr + 16)), c_at(par, rt, ks)[lane], acc);
            }
          }
          const float sr = Sl[par * RWS + rt * 16 + lr];
#pragma unroll
          for (int q = 0; q < 4; ++q) os[rt][q] = ge[q] * (sr * acc[q]);
        }
      }
      // ---- this wave's Q rows of the next chunk (the loads are unconditional,
      //      the chunk index clamped, so the in-order load counter never has to
      //      assume the shorter path)
      if (c + 1 < NC) stage_q();
      load_q(c + 2 < NC ? c + 2 : NC - 1);
      __syncthreads();
    }
    if (NC > 0) output(NC - 1);
    return;
  }

  // ================================================================ staging waves
  const int st = tid - 4 * 64;  // 0 .. 127
  const uint16_t* const k_c0 = stg0 ? a.sm.sk : a.k;
  const uint16_t* const v_c0 = stg0 ? a.sm.sv : a.v;
  const float* const b_c0 = stg0 ? a.sm.sb : a.beta;
  const size_t wsc = size_t(a.sm.chunk0(bs)) * a.H + h;  // workspace index of the first chunk
  // K: units u = st + 128 m (m < 4) of token pair u % 32 and dims [8 (u / 32), +8);
  // T: granules st + 128 m (m < 8) of the chunk's 960; V: token pair st % 32,
  // rows [8 (st / 32), +8) of the block; g and beta: token st % 64
  u32x4 kw[4][2], tw[8], vw[2];
  float gv = 0.f, bv = 0.f;
  int kc = 0;  // the chunk the registers hold
  auto load_in = [&](int c) {
    kc = c;
    const size_t crow = chunk_row(c);
    const uint16_t* kb = (c == 0 ? k_c0 : a.k) + crow * HD + size_t(h) * PD;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int u = st + 128 * m, p = u & 31, s8 = (u >> 5) * 8;
      kw[m][0] = *reinterpret_cast<const u32x4*>(kb + in_row(c, 2 * p) * HD32 + s8);
      kw[m][1] = *reinterpret_cast<const u32x4*>(kb + in_row(c, 2 * p + 1) * HD32 + s8);
    }
    const __bf16* tb = a.T_ws + (wsc + size_t(c) * a.H) * (3 * TT * 256);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int gi = st + 128 * m < 3 * TT * 32 ? st + 128 * m : 3 * TT * 32 - 1;
      tw[m] = *reinterpret_cast<const u32x4*>(tb + gi * 8);
    }
    const int p = st & 31;
    const uint16_t* vb = (c == 0 ? v_c0 : a.v) + crow * HD + size_t(h) * PD + r0 + 8 * (st >> 5);
    vw[0] = *reinterpret_cast<const u32x4*>(vb + in_row(c, 2 * p) * HD32);
    vw[1] = *reinterpret_cast<const u32x4*>(vb + in_row(c, 2 * p + 1) * HD32);
    gv = a.g_ws[(wsc + size_t(c) * a.H) * PC + (st & 63)];
    const float* bb = (c == 0 ? b_c0 : a.beta) + crow * a.H + h;
    bv = bb[in_row(c, st & 63) * uint32_t(a.H)];
  };
  auto stage_in = [&](int par) {
    __bf16* K = Kl + par * PC * KP;
    uint32_t* kt = reinterpret_cast<uint32_t*>(KTl + par * PD * PC);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int u = st + 128 * m, p = u & 31, s8 = (u >> 5) * 8;
      const u32x4 w0 = tok_ok(kc, 2 * p) ? kw[m][0] : z4;  // padding keys are 0
      const u32x4 w1 = tok_ok(kc, 2 * p + 1) ? kw[m][1] : z4;
      *reinterpret_cast<u32x4*>(K + (2 * p) * KP + s8) = w0;
      *reinterpret_cast<u32x4*>(K + (2 * p + 1) * KP + s8) = w1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // K^T dword: tokens (2 p, 2 p + 1) of dim s8 + e
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        kt[kt_index(s8 + e, 2 * p) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      }
    }
    __bf16* T = Tl + par * 3 * TT * 256;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (st + 128 * m < 3 * TT * 32) *reinterpret_cast<u32x4*>(T + (st + 128 * m) * 8) = tw[m];
    {  // V^T dwords: rows 8 (st / 32) + e, tokens (2 p, 2 p + 1)
      const int p = st & 31, o = st >> 5;
      const u32x4 w0 = tok_ok(kc, 2 * p) ? vw[0] : z4, w1 = tok_ok(kc, 2 * p + 1) ? vw[1] : z4;
      uint32_t* vt = reinterpret_cast<uint32_t*>(Vl + par * RWS * VTP);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        vt[((8 * o + e) * VTP + 2 * p) >> 1] = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      }
    }
    if (wave == 4) {  // per-token scalars, lane = token (padding: beta = 0)
      float* F = Fl + par * 4 * PC;
      const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 63));
      F[lane] = gv;
      F[PC + lane] = expf(gv);
      F[2 * PC + lane] = tok_ok(kc, lane) ? bv : 0.f;
      F[3 * PC + lane] = expf(gC - gv);
    }
  };
  if (NC > 0) {
    load_in(0);
    stage_in(0);
    load_in(NC > 1 ? 1 : 0);
  }
  __syncthreads();
  for (int c = 0; c < NC; ++c) {
    if (c + 1 < NC) stage_in((c + 1) & 1);
    load_in(c + 2 < NC ? c + 2 : NC - 1);
    __syncthreads();
  }
}

// Chunks the workspace holds: B ceil(T / 64) for uniform lengths; for
// variable lengths summing to N new tokens, sum ceil(n / 64) <= floor(N / 64)
// + B, and with a buffered prefix of at most 63 writes per sequence,
// sum ceil((pre + n) / 64) <= floor(N / 64) + 2 B.
static size_t gdn_new_tokens(const PrefillLaunch& L) { return L.varlen ? size_t(L.T) : size_t(L.B) * L.T; }
// Shapes the chunk kernels do not take directly run on padded copies in the
// workspace:
//   * d_k = d_v = 64: the head runs as a d = 128 head whose extra key
//     dimensions and value rows are zero.  Keys padded with zeros get and
//     erase nothing in the extra columns, zero value rows write nothing, and
//     every product and row absmax only gains +0 terms, so the padded head
//     carries the d = 64 state exactly in its first 64 rows and columns.
//   * a window W that is not a multiple of 64 tokens: every window becomes
//     Wp = 64 ceil(W / 64) positions whose last Wp - W are writes that change
//     nothing (k = q = v = 0, alpha = 1, beta = 0): the state passes them
//     unchanged, so the end of every Wp / 64-th chunk is exactly a window's
//     end and is requantized there.  A state that is never requantized runs
//     as one window of all T tokens.
// gdn_pad_kernel builds the padded q, k, v (and alpha, beta; and the stored
// state at d = 64); gdn_unpad_kernel copies the real tokens' outputs (and the
// final state at d = 64) back.
struct PadArgs {
  const uint16_t* x[3];  // q, k, v [B][T][H][ds] bf16
  uint16_t* y[3];        // [B][Tp][H][128] bf16
  const float* a;        // alpha, beta [B][T][H] (NULL: not padded, W = 64)
  const float* be;
  float* pa;             // [B][Tp][H]
  float* pb;
  int64_t B, T, H;
  int W, Wp, ds;         // window, its padded positions (a multiple of 64), source width
  const int8_t* c0;      // stored state [bh][64][RB64] (NULL: zero state or not padded)
  const float* s0;       // [bh][64]
  int8_t* pc0;           // [bh][128][RB128]
  float* ps0;            // [bh][128]
  int64_t bh;
  int rb64;              // bytes per stored row at d = 64: 64 (8-bit) or 32 (4-bit)
};

// Positions of a padded sequence: its whole windows of Wp positions, then the
// T mod W tokens of an open last window (the hand-over) unpadded.
__device__ __forceinline__ int64_t padded_len(int64_t T, int W, int Wp) { return T / W * Wp + T % W; }

__global__ __launch_bounds__(256) void gdn_pad_kernel(PadArgs a) {
  const int64_t Tp = padded_len(a.T, a.W, a.Wp);
  const int64_t rows = a.B * Tp * a.H;  // padded rows
  const int64_t stride = int64_t(gridDim.x) * 256;
  const int gs = a.ds / 8;  // 16-byte granules per source row
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < rows * 48; e += stride) {
    const int64_t r = e / 48;  // padded row (b Tp + p) H + h
    const int op = int(e % 48) / 16, g = int(e % 16);
    const int64_t h = r % a.H, bp = r / a.H, p = bp % Tp, b = bp / Tp;
    const int i = int(p % a.Wp);  // position in its window
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (i < a.W && g < gs) {
      const int64_t t = p / a.Wp * a.W + i;  // the source token
      w = reinterpret_cast<const uint4*>(a.x[op] + ((b * a.T + t) * a.H + h) * a.ds)[g];
    }
    reinterpret_cast<uint4*>(a.y[op] + r * PD)[g] = w;
  }
  if (a.a) {
    for (int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x; r < rows; r += stride) {
      const int64_t h = r % a.H, bp = r / a.H, p = bp % Tp, b = bp / Tp;
      const int i = int(p % a.Wp);
      float al = 1.f, bt = 0.f;
      if (i < a.W) {
        const int64_t src = (b * a.T + p / a.Wp * a.W + i) * a.H + h;
        al = a.a[src];
        bt = a.be[src];
      }
      a.pa[r] = al;
      a.pb[r] = bt;
    }
  }
  if (!a.pc0) return;
  const int rb128 = 2 * a.rb64;
  const int64_t ns = a.bh * PD * (rb128 / 16);
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ns; e += stride) {
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
  const char* po;  // [B][Tp][H][128] outputs (eo bytes each)
  char* o;         // [B][T][H][ds]
  int64_t B, T, H;
  int W, Wp, ds, eo;
  const int8_t* pc;  // [bh][128][RB128] (NULL: no padded codes to copy back)
  const float* ps;
  int8_t* c;         // [bh][64][RB64]
  float* sc;
  const float* psf;  // fp32 state [bh][128][128] (NULL: none to copy back)
  float* sf;         // [bh][64][64]
  int64_t bh;
  int rb64;
};

__global__ __launch_bounds__(256) void gdn_unpad_kernel(UnpadArgs a) {
  const int gpr = a.ds * a.eo / 16;  // 16-byte granules per output row
  const int64_t Tp = padded_len(a.T, a.W, a.Wp);
  const int64_t n = a.B * a.T * a.H * gpr;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += stride) {
    const int64_t row = e / gpr;  // (b T + t) H + h
    const int g = int(e % gpr);
    const int64_t h = row % a.H, bt = row / a.H, t = bt % a.T, b = bt / a.T;
    const int64_t prow = (b * Tp + t / a.W * a.Wp + t % a.W) * a.H + h;
    reinterpret_cast<uint4*>(a.o + row * a.ds * a.eo)[g] = reinterpret_cast<const uint4*>(a.po + prow * PD * a.eo)[g];
  }
  if (a.psf) {
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < a.bh * 64 * 16; e += stride) {
      const int64_t r = e / 16;  // bh * 64 + row
      const int g = int(e % 16);
      const int64_t bh = r / 64, rr = r % 64;
      reinterpret_cast<float4*>(a.sf + r * 64)[g] = reinterpret_cast<const float4*>(a.psf + (bh * PD + rr) * PD)[g];
    }
  }
  if (!a.pc) return;
  const int64_t ns = a.bh * 64 * (a.rb64 / 16);
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ns; e += stride) {
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
static size_t gdn_ws_T(const PrefillLaunch& L) { return gdn_chunks(L) * L.H * 3 * TT * 256 * 2; }
static size_t gdn_ws_g(const PrefillLaunch& L) { return gdn_chunks(L) * L.H * PC * 4; }
// staged chunk 0 when resuming: k, q, v bf16 [B][64][H][128], alpha, beta fp32 [B][64][H]
static size_t gdn_ws_stage(const PrefillLaunch& L) {
  return L.resume ? size_t(L.B) * PC * L.H * (3 * PD * 2 + 2 * 4) : 0;
}
static bool gdn_mapped(const PrefillLaunch& L) { return L.varlen || L.resume; }
static size_t gdn_ws_map(const PrefillLaunch& L) { return gdn_mapped(L) ? (4 * size_t(L.B) + 2) * 4 : 0; }
// rotated q and k (GDNQ_FLAG_WHT, whole windows only): [2][B*T*H][128] bf16
// token rows of q and k: B T H, or T H packed tokens (variable lengths)
static size_t gdn_token_rows(const PrefillLaunch& L) { return (L.varlen ? size_t(1) : size_t(L.B)) * L.T * L.H; }
static size_t gdn_ws_rot(const PrefillLaunch& L) { return L.wht ? 2 * gdn_token_rows(L) * PD * 2 : 0; }
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
// Window-buffer formats of decode: 0 fp32, 1 bf16, 2 FP8 vector pairs (E4M3
// codes; one fp32 scale per vector after all the codes).
struct StageArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  const void* buf_k;
  const void* buf_v;
  const float* buf_ks;  // FP8: the vectors' scales
  const float* buf_vs;
  int fmt;
  const float* buf_alpha;
  const float* buf_beta;
  uint16_t* sk;
  uint16_t* sq;
  uint16_t* sv;
  float* sa;
  float* sb;
  SeqMap sm;
  int B, H, W;
  int ds;  // elements of a buffered key / value (64 or 128; staged rows hold 128, zero past ds)
};

__global__ __launch_bounds__(256) void gdn_stage_kernel(StageArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int pre = a.sm.npre(b), n = a.sm.ntok(b);
  const size_t tok0 = a.sm.tok0(b);
  const size_t HD = size_t(a.H) * PD;
  for (int e = threadIdx.x; e < PC * PD / 2; e += 256) {  // two dims per thread
    const int pos = e / (PD / 2), d = 2 * (e % (PD / 2));
    uint32_t kw = 0u, qw = 0u, vw = 0u;
    if (pos < pre) {  // a buffered write enters at bf16 (exact for bf16 inputs); zero past ds
      if (d < a.ds) {
        const size_t slot = size_t(bh) * a.W + pos, src = slot * a.ds + d;
        if (a.fmt == 1) {
          kw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.buf_k) + src);
          vw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.buf_v) + src);
        } else {
          float2 kf, vf;
          if (a.fmt == 2) {  // the stored value: code * scale in fp32
            const float2 kc = e4m3_unpack2(*reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.buf_k) + src), false);
            const float2 vc = e4m3_unpack2(*reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.buf_v) + src), false);
            const float ks = a.buf_ks[slot], vs = a.buf_vs[slot];
            kf = make_float2(kc.x * ks, kc.y * ks);
            vf = make_float2(vc.x * vs, vc.y * vs);
          } else {
            kf = *reinterpret_cast<const float2*>(static_cast<const float*>(a.buf_k) + src);
            vf = *reinterpret_cast<const float2*>(static_cast<const float*>(a.buf_v) + src);
          }
          kw = f32_to_bf16_bits(kf.x) | (f32_to_bf16_bits(kf.y) << 16);
          vw = f32_to_bf16_bits(vf.x) | (f32_to_bf16_bits(vf.y) << 16);
        }
      }
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
// (keys in the state's basis; fp32, bf16 -- the bf16 inputs themselves -- or
// FP8 vector pairs encoded as decode's append does: scale = absmax / 448 and
// codes nearest to x / scale, IEEE divisions, ties to even) and its fill
// becomes r.  Slots that
// already hold a buffered prefix write (when resuming, before any window
// closed) are left as they are.  One workgroup per (sequence, head).
struct HandoffArgs {
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  void* buf_k;
  void* buf_v;
  float* buf_ks;  // FP8: the vectors' scales
  float* buf_vs;
  int fmt;
  float* buf_alpha;
  float* buf_beta;
  int32_t* fill_out;
  SeqMap sm;
  int B, H, W;  // W: decode's window (buffer slots per head)
  int ds;       // elements of a buffered key / value (64 or 128; the source rows hold 128)
};

__global__ __launch_bounds__(256) void gdn_handoff_kernel(HandoffArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int len = a.sm.len(b), pre = a.sm.npre(b);
  const int r = len % PC;
  const int p0 = len - r;  // position of slot 0
  const int s0 = max(pre - p0, 0);  // first slot that takes a new token
  const size_t t0 = a.sm.tok0(b);
  // 8 dims per thread: a slot's ds / 8 threads are consecutive lanes (the
  // stride 256 is a multiple of that), so an FP8 vector's absmax is a 16- or
  // 8-lane reduction inside one wave
  const int per = a.ds / 8;
  for (int e = threadIdx.x; e < (r - s0) * per; e += 256) {
    const int slot = s0 + e / per, d = 8 * (e % per);
    const size_t src = ((t0 + (p0 + slot - pre)) * a.H + h) * PD + d;
    const size_t sl = size_t(bh) * a.W + slot, dst = sl * a.ds + d;
    const uint4 kw = *reinterpret_cast<const uint4*>(a.k + src);
    const uint4 vw = *reinterpret_cast<const uint4*>(a.v + src);
    if (a.fmt == 1) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.buf_k) + dst) = kw;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.buf_v) + dst) = vw;
      continue;
    }
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, vv[4] = {vw.x, vw.y, vw.z, vw.w};
    float kf[8], vf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kf[2 * i] = bf16_lo(kk[i]);
      kf[2 * i + 1] = bf16_hi(kk[i]);
      vf[2 * i] = bf16_lo(vv[i]);
      vf[2 * i + 1] = bf16_hi(vv[i]);
    }
    if (a.fmt == 2) {
      float mk = 0.f, mv = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mk = fmaxf(mk, fabsf(kf[i]));
        mv = fmaxf(mv, fabsf(vf[i]));
      }
      mk = per == 16 ? group_max<16>(mk) : group_max<8>(mk);
      mv = per == 16 ? group_max<16>(mv) : group_max<8>(mv);
      const float sk = __fdiv_rn(mk, 448.f);
      const float sv = __fdiv_rn(mv, 448.f);
      uint32_t ck[2], cv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float c[4], w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = sk > 0.f ? e4m3_round(__fdiv_rn(kf[4 * i + j], sk)) : 0.f;
          w[j] = sv > 0.f ? e4m3_round(__fdiv_rn(vf[4 * i + j], sv)) : 0.f;
        }
        ck[i] = e4m3_pack2(c[0], c[1]) | (e4m3_pack2(c[2], c[3]) << 16);
        cv[i] = e4m3_pack2(w[0], w[1]) | (e4m3_pack2(w[2], w[3]) << 16);
      }
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.buf_k) + dst) = make_uint2(ck[0], ck[1]);
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(a.buf_v) + dst) = make_uint2(cv[0], cv[1]);
      if (d == 0) {
        a.buf_ks[sl] = sk;
        a.buf_vs[sl] = sv;
      }
      continue;
    }
    float* bk = static_cast<float*>(a.buf_k) + dst;
    float* bv = static_cast<float*>(a.buf_v) + dst;
    *reinterpret_cast<float4*>(bk) = make_float4(kf[0], kf[1], kf[2], kf[3]);
    *reinterpret_cast<float4*>(bk + 4) = make_float4(kf[4], kf[5], kf[6], kf[7]);
    *reinterpret_cast<float4*>(bv) = make_float4(vf[0], vf[1], vf[2], vf[3]);
    *reinterpret_cast<float4*>(bv + 4) = make_float4(vf[4], vf[5], vf[6], vf[7]);
  }
  for (int slot = s0 + threadIdx.x; slot < r; slot += 256) {
    const size_t src = (t0 + (p0 + slot - pre)) * a.H + h;
    a.buf_alpha[size_t(bh) * a.W + slot] = a.alpha[src];
    a.buf_beta[size_t(bh) * a.W + slot] = a.beta[src];
  }
  if (h == 0 && threadIdx.x == 0) a.fill_out[b] = r;
}

// ---- padded runs of packed (variable-length) or resumed sequences
// Sequence b has f_b buffered writes (resuming; none otherwise) and n_b new
// tokens: P_b = f_b + n_b positions in windows of W from its first buffered
// write.  Its padded run has P_b / W whole windows of 64 positions (W writes,
// then 64 - W that change nothing) and the P_b mod W positions of the open
// window; the f_b buffered positions are staged from decode's buffer as
// always, so it takes Np_b = 64 (P_b / W) + P_b mod W - f_b padded token rows.
__device__ __forceinline__ int padded_token_rows(int n, int f, int W) {
  const int P = f + n;
  return P / W * PC + P % W - f;
}

// last b in [0, B] with off[b] <= r (off ascending from off[0] = 0)
__device__ __forceinline__ int seq_of(const int32_t* off, int B, int64_t r) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One workgroup: token offsets tok[0..B] (cu sanitized as the sequence map
// does it: the running maximum of cu clamped to [0, T]; uniform: b T),
// buffered writes pre[b] = fill clamped to [0, W - 1] (or 0) and padded row
// offsets cup[0..B] (exclusive sums of Np_b).
struct PadMapArgs {
  const int32_t* cu;    // [B+1] token offsets, or nullptr: T tokens per sequence
  const int32_t* fill;  // [B] buffered writes, or nullptr
  int32_t* tok;         // [B+1]
  int32_t* cup;         // [B+1]
  int32_t* pre;         // [B]
  int B, T, W;
};

__global__ __launch_bounds__(1024) void gdn_padmap_kernel(PadMapArgs a) {
  __shared__ int32_t sv[1025];
  __shared__ int32_t sc[1024];
  const int t = threadIdx.x;
  auto off = [&](int i) { return a.cu ? min(max(a.cu[i], 0), a.T) : i * a.T; };
  int carry_tok = 0, carry_p = 0;
  for (int base = 0; base <= a.B; base += 1024) {
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
    const int f = i < a.B && a.fill ? min(max(a.fill[i], 0), a.W - 1) : 0;
    const int np = i < a.B ? padded_token_rows(sv[t + 1] - sv[t], f, a.W) : 0;
    sc[t] = np;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int y = t >= o ? sc[t - o] : 0;
      __syncthreads();
      sc[t] += y;
      __syncthreads();
    }
    if (i <= a.B) {
      a.tok[i] = sv[t];
      a.cup[i] = carry_p + sc[t] - np;
    }
    if (i < a.B) a.pre[i] = f;
    carry_tok = sv[1023];
    carry_p += sc[1023];
    __syncthreads();
  }
}

// Padded token rows [Tp][H][128] (and alpha, beta [Tp][H]) from the token rows
// [.][H][ds]: row cup[b] + j of sequence b is position p = f_b + j of its
// padded run; rows past cup[B] are zero.
struct MapPadArgs {
  const uint16_t* x[3];
  uint16_t* y[3];
  const float* a;
  const float* be;
  float* pa;
  float* pb;
  const int32_t* tok;
  const int32_t* cup;
  const int32_t* pre;
  int64_t Tp;
  int B, H, W, ds;
};

__device__ __forceinline__ int64_t padded_source(const MapPadArgs& a, int64_t rp) {  // token row, or -1
  if (rp >= a.cup[a.B]) return -1;
  const int b = seq_of(a.cup, a.B, rp);
  const int f = a.pre[b], n = a.tok[b + 1] - a.tok[b];
  const int p = f + int(rp - a.cup[b]);
  const int nw = (f + n) / a.W, w = p / PC, i = p % PC;
  if (w < nw && i >= a.W) return -1;  // a padding write of a whole window
  return int64_t(a.tok[b]) + (w < nw ? w * a.W + i : nw * a.W + i) - f;
}

__global__ __launch_bounds__(256) void gdn_mappad_kernel(MapPadArgs a) {
  const int64_t rows = a.Tp * a.H;
  const int64_t stride = int64_t(gridDim.x) * 256;
  const int gs = a.ds / 8;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < rows * 48; e += stride) {
    const int64_t r = e / 48;  // padded row rp H + h
    const int op = int(e % 48) / 16, g = int(e % 16);
    const int64_t h = r % a.H, src = padded_source(a, r / a.H);
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (src >= 0 && g < gs) w = reinterpret_cast<const uint4*>(a.x[op] + (src * a.H + h) * a.ds)[g];
    reinterpret_cast<uint4*>(a.y[op] + r * PD)[g] = w;
  }
  for (int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x; r < rows; r += stride) {
    const int64_t h = r % a.H, src = padded_source(a, r / a.H);
    a.pa[r] = src >= 0 ? a.a[src * a.H + h] : 1.f;
    a.pb[r] = src >= 0 ? a.be[src * a.H + h] : 0.f;
  }
}

// Outputs of the token rows back from the padded rows: token tok[b] + j is
// position p = f_b + j, padded position 64 (p / W) + p mod W.
struct MapUnpadArgs {
  const char* po;  // [Tp][H][128] (eo bytes each)
  char* o;         // [rows][H][ds]
  const int32_t* tok;
  const int32_t* cup;
  const int32_t* pre;
  int64_t rows;    // token rows the output holds
  int B, H, W, ds, eo;
};

__global__ __launch_bounds__(256) void gdn_mapunpad_kernel(MapUnpadArgs a) {
  const int gpr = a.ds * a.eo / 16;
  const int64_t n = a.rows * a.H * gpr, stride = int64_t(gridDim.x) * 256;
  const int32_t T_all = a.tok[a.B];
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += stride) {
    const int64_t row = e / gpr;  // t H + h
    const int g = int(e % gpr);
    const int64_t h = row % a.H, t = row / a.H;
    if (t >= T_all) continue;  // past the (sanitized) sequences: not an output of any
    const int b = seq_of(a.tok, a.B, t);
    const int f = a.pre[b], p = f + int(t - a.tok[b]);
    const int64_t prow = (int64_t(a.cup[b]) + p / a.W * PC + p % a.W - f) * a.H + h;
    reinterpret_cast<uint4*>(a.o + row * a.ds * a.eo)[g] = reinterpret_cast<const uint4*>(a.po + prow * PD * a.eo)[g];
  }
}

static size_t gdn_ws_128(const PrefillLaunch& L) {
  return gdn_ws_T(L) + gdn_ws_g(L) + gdn_ws_stage(L) + gdn_ws_map(L) + gdn_ws_rot(L);
}
// The window in tokens (a state never requantized: all T tokens as one) and
// its padded length, a multiple of the 64-position chunk.
static int gdn_window(const PrefillLaunch& L) { return L.no_requant ? (L.T > 0 ? L.T : PC) : L.W; }
static int gdn_window_padded(const PrefillLaunch& L) { return (gdn_window(L) + PC - 1) / PC * PC; }
// The padded run: d = 128, windows of whole 64-position chunks.
static bool gdn_padded(const PrefillLaunch& L) { return L.d_k == 64 || gdn_window(L) % PC != 0; }
static PrefillLaunch gdn_padded_launch(const PrefillLaunch& L) {
  PrefillLaunch L2 = L;
  L2.d_k = L2.d_v = PD;
  L2.T = L.T / gdn_window(L) * gdn_window_padded(L) + L.T % gdn_window(L);
  L2.W = gdn_window_padded(L);
  L2.C = PC;
  return L2;
}
struct PadLayout {
  size_t qkv, ab, c0, s0, o, c, sc, sf, inner, total;
};
static PadLayout gdn_pad_layout(const PrefillLaunch& L) {
  const PrefillLaunch L2 = gdn_padded_launch(L);
  const size_t rows = size_t(L.B) * L2.T * L.H, bh = size_t(L.B) * L.H;
  const size_t rb = L.q4 ? PD / 2 : PD, eo = L.out_bf16 ? 2 : 4;
  const bool pad_ab = gdn_window(L) % PC != 0, pad_state = L.d_k == 64;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  PadLayout p{};
  p.qkv = 0;
  p.ab = p.qkv + up(3 * rows * PD * 2);
  p.c0 = p.ab + (pad_ab ? up(2 * rows * 4) : 0);
  p.s0 = p.c0 + (pad_state ? up(bh * PD * rb) : 0);
  p.o = p.s0 + (pad_state ? up(bh * PD * 4) : 0);
  p.c = p.o + up(rows * PD * eo);
  p.sc = p.c + (pad_state && !L.no_requant ? up(bh * PD * rb) : 0);
  p.sf = p.sc + (pad_state && !L.no_requant ? up(bh * PD * 4) : 0);
  p.inner = p.sf + (pad_state && L.no_requant ? up(bh * PD * PD * 4) : 0);
  p.total = p.inner + gdn_ws_128(L2);
  return p;
}

// Packed / resumed sequences padded: the padded rows' upper bound, sum over
// sequences of 64 (f_b + n_b) / W - f_b <= 64 (N + B (W - 1)) / W.
static int64_t gdn_map_rows(const PrefillLaunch& L) {
  const int64_t N = L.varlen ? int64_t(L.T) : int64_t(L.B) * L.T;  // new tokens
  const int64_t pre_max = L.resume ? int64_t(L.B) * (L.W - 1) : 0;
  return (PC * (N + pre_max) + L.W - 1) / L.W;
}
static bool gdn_map_padded(const PrefillLaunch& L) { return (L.varlen || L.resume) && gdn_padded(L); }
static PrefillLaunch gdn_map_launch(const PrefillLaunch& L) {
  PrefillLaunch L2 = L;
  L2.d_k = L2.d_v = PD;
  L2.T = int(gdn_map_rows(L));
  L2.W = L2.C = PC;
  L2.varlen = true;  // packed: the padded lengths differ between sequences
  return L2;
}
struct MapLayout {
  size_t qkv, ab, c0, s0, o, c, sc, map, inner, total;
};
static MapLayout gdn_map_layout(const PrefillLaunch& L) {
  const PrefillLaunch L2 = gdn_map_launch(L);
  const size_t rows = size_t(L2.T) * L.H, bh = size_t(L.B) * L.H;
  const size_t rb = L.q4 ? PD / 2 : PD, eo = L.out_bf16 ? 2 : 4;
  const bool pad_state = L.d_k == 64;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  MapLayout p{};
  p.qkv = 0;
  p.ab = p.qkv + up(3 * rows * PD * 2);
  p.c0 = p.ab + up(2 * rows * 4);
  p.s0 = p.c0 + (pad_state ? up(bh * PD * rb) : 0);
  p.o = p.s0 + (pad_state ? up(bh * PD * 4) : 0);
  p.c = p.o + up(rows * PD * eo);
  p.sc = p.c + (pad_state ? up(bh * PD * rb) : 0);
  p.map = p.sc + (pad_state ? up(bh * PD * 4) : 0);
  p.inner = p.map + up((3 * size_t(L.B) + 2) * 4);
  p.total = p.inner + gdn_ws_128(L2);
  return p;
}

size_t prefill_gdn_workspace_bytes(const PrefillLaunch& L) {
  if (gdn_map_padded(L)) return gdn_map_layout(L).total;
  if (gdn_padded(L)) return gdn_pad_layout(L).total;
  return gdn_ws_128(L);
}

static hipError_t launch_prefill_gdn_mapped_padded(const PrefillLaunch& L, hipStream_t stream);

static hipError_t launch_prefill_gdn128(const PrefillLaunch& Lin, hipStream_t stream);

hipError_t launch_prefill_gdn(const PrefillLaunch& L, hipStream_t stream) {
  if (gdn_map_padded(L)) return launch_prefill_gdn_mapped_padded(L, stream);
  if (!gdn_padded(L)) return launch_prefill_gdn128(L, stream);
  // pad, run the d = 128, 64-chunk kernels on the workspace copies, unpad
  const PadLayout P = gdn_pad_layout(L);
  const PrefillLaunch L2p = gdn_padded_launch(L);
  char* ws = static_cast<char*>(L.workspace);
  const int64_t rows = int64_t(L.B) * L2p.T * L.H, bh = int64_t(L.B) * L.H;
  const bool pad_ab = gdn_window(L) % PC != 0, pad_state = L.d_k == 64;
  const int Wt = gdn_window(L), Wp = gdn_window_padded(L);
  const int rb64 = L.q4 ? 32 : 64;
  uint16_t* pq = reinterpret_cast<uint16_t*>(ws + P.qkv);
  float* pal = reinterpret_cast<float*>(ws + P.ab);
  PadArgs pa{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v)},
             {pq, pq + rows * PD, pq + 2 * rows * PD},
             pad_ab ? L.alpha : nullptr, pad_ab ? L.beta : nullptr, pad_ab ? pal : nullptr, pad_ab ? pal + rows : nullptr,
             L.B, L.T, L.H, Wt, Wp, L.d_k,
             pad_state ? L.init_codes : nullptr, L.init_scales,
             pad_state && L.init_codes ? reinterpret_cast<int8_t*>(ws + P.c0) : nullptr,
             reinterpret_cast<float*>(ws + P.s0), bh, rb64};
  const int64_t work = rows * 48 > bh * PD * 8 ? rows * 48 : bh * PD * 8;
  const unsigned grid = unsigned(work / 256 + 1 < 4096 ? work / 256 + 1 : 4096);
  hipLaunchKernelGGL(gdn_pad_kernel, dim3(grid), dim3(256), 0, stream, pa);
  if (hipError_t e = hipGetLastError()) return e;
  PrefillLaunch L2 = L2p;
  L2.q = pa.y[0];
  L2.k = pa.y[1];
  L2.v = pa.y[2];
  if (pad_ab) {
    L2.alpha = pa.pa;
    L2.beta = pa.pb;
  }
  if (pad_state) {
    L2.init_codes = pa.pc0;
    L2.init_scales = L.init_codes ? pa.ps0 : nullptr;
    if (L.no_requant) {
      L2.state_f32 = reinterpret_cast<float*>(ws + P.sf);
    } else {
      L2.codes = reinterpret_cast<int8_t*>(ws + P.c);
      L2.scales = reinterpret_cast<float*>(ws + P.sc);
    }
  }
  L2.o = ws + P.o;
  L2.workspace = ws + P.inner;
  if (hipError_t e = launch_prefill_gdn128(L2, stream)) return e;
  const bool back_codes = pad_state && !L.no_requant, back_f32 = pad_state && L.no_requant;
  UnpadArgs ua{ws + P.o, static_cast<char*>(L.o), L.B, L.T, L.H, Wt, Wp, L.d_k, L.out_bf16 ? 2 : 4,
               back_codes ? L2.codes : nullptr, L2.scales, L.codes, L.scales,
               back_f32 ? L2.state_f32 : nullptr, L.state_f32, bh, rb64};
  hipLaunchKernelGGL(gdn_unpad_kernel, dim3(grid), dim3(256), 0, stream, ua);
  return hipGetLastError();
}

// Packed or resumed sequences at d = 64 or with decode's window below 64:
// map and pad every sequence, run the d = 128, 64-chunk kernels on the packed
// padded rows (the hand-over writes decode's W-slot buffer of d elements),
// then copy the outputs (and the d = 64 state) back.
static hipError_t launch_prefill_gdn_mapped_padded(const PrefillLaunch& L, hipStream_t stream) {
  const MapLayout P = gdn_map_layout(L);
  const PrefillLaunch L2p = gdn_map_launch(L);
  char* ws = static_cast<char*>(L.workspace);
  const int64_t Tp = L2p.T, rows = Tp * L.H, bh = int64_t(L.B) * L.H;
  const bool pad_state = L.d_k == 64;
  const int rb64 = L.q4 ? 32 : 64;
  int32_t* tok = reinterpret_cast<int32_t*>(ws + P.map);
  int32_t* cup = tok + (L.B + 1);
  int32_t* pre = cup + (L.B + 1);
  PadMapArgs m{L.cu_seqlens, L.resume ? L.fill_in : nullptr, tok, cup, pre, L.B, L.T, L.W};
  hipLaunchKernelGGL(gdn_padmap_kernel, dim3(1), dim3(1024), 0, stream, m);
  if (hipError_t e = hipGetLastError()) return e;
  uint16_t* pq = reinterpret_cast<uint16_t*>(ws + P.qkv);
  float* pal = reinterpret_cast<float*>(ws + P.ab);
  MapPadArgs pa{{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v)},
                {pq, pq + rows * PD, pq + 2 * rows * PD}, L.alpha, L.beta, pal, pal + rows,
                tok, cup, pre, Tp, L.B, L.H, L.W, L.d_k};
  const int64_t work = rows * 48;
  const unsigned grid = unsigned(work / 256 + 1 < 4096 ? work / 256 + 1 : 4096);
  hipLaunchKernelGGL(gdn_mappad_kernel, dim3(grid), dim3(256), 0, stream, pa);
  if (hipError_t e = hipGetLastError()) return e;
  PrefillLaunch L2 = L2p;
  L2.q = pa.y[0];
  L2.k = pa.y[1];
  L2.v = pa.y[2];
  L2.alpha = pa.pa;
  L2.beta = pa.pb;
  L2.cu_seqlens = cup;
  L2.fill_in = L.resume ? pre : nullptr;
  if (pad_state) {  // the stored state widened to d = 128 (rows and columns past 64 zero)
    PadArgs sp{{nullptr, nullptr, nullptr}, {nullptr, nullptr, nullptr}, nullptr, nullptr, nullptr, nullptr,
               0, 0, 1, 1, PC, L.d_k, L.init_codes, L.init_scales,
               L.init_codes ? reinterpret_cast<int8_t*>(ws + P.c0) : nullptr,
               reinterpret_cast<float*>(ws + P.s0), bh, rb64};
    if (L.init_codes) {
      hipLaunchKernelGGL(gdn_pad_kernel, dim3(unsigned(bh * PD * 8 / 256 + 1 < 4096 ? bh * PD * 8 / 256 + 1 : 4096)),
                         dim3(256), 0, stream, sp);
      if (hipError_t e = hipGetLastError()) return e;
    }
    L2.init_codes = sp.pc0;
    L2.init_scales = L.init_codes ? sp.ps0 : nullptr;
    L2.codes = reinterpret_cast<int8_t*>(ws + P.c);
    L2.scales = reinterpret_cast<float*>(ws + P.sc);
  }
  L2.o = ws + P.o;
  L2.workspace = ws + P.inner;
  if (hipError_t e = launch_prefill_gdn128(L2, stream)) return e;
  const int64_t out_rows = L.varlen ? int64_t(L.T) : int64_t(L.B) * L.T;
  MapUnpadArgs ua{ws + P.o, static_cast<char*>(L.o), tok, cup, pre, out_rows, L.B, L.H, L.W, L.d_k,
                  L.out_bf16 ? 2 : 4};
  const int64_t uwork = out_rows * L.H * (L.d_k * (L.out_bf16 ? 2 : 4) / 16);
  if (uwork > 0) {
    hipLaunchKernelGGL(gdn_mapunpad_kernel, dim3(unsigned(uwork / 256 + 1 < 4096 ? uwork / 256 + 1 : 4096)),
                       dim3(256), 0, stream, ua);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (pad_state) {
    UnpadArgs us{nullptr, nullptr, 0, 0, 1, 1, PC, L.d_k, 1, L2.codes, L2.scales, L.codes, L.scales, nullptr, nullptr,
                 bh, rb64};
    hipLaunchKernelGGL(gdn_unpad_kernel, dim3(unsigned(bh * 64 * 4 / 256 + 1)), dim3(256), 0, stream, us);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

static int gdn_buf_fmt(const PrefillLaunch& L) { return L.buf_fp8 ? 2 : L.buf_bf16 ? 1 : 0; }
// FP8 window buffer: the fp32 scales follow the B H W d code bytes
static float* gdn_fp8_scales(const PrefillLaunch& L, void* codes) {
  return L.buf_fp8 ? reinterpret_cast<float*>(static_cast<uint8_t*>(codes) + size_t(L.B) * L.H * L.buf_W * L.buf_d)
                   : nullptr;
}

static hipError_t launch_prefill_gdn128(const PrefillLaunch& Lin, hipStream_t stream) {
  PrefillLaunch L = Lin;
  char* ws = static_cast<char*>(L.workspace);
  if (L.wht && L.B > 0 && L.T > 0) {  // rotate q and k once; the chunk kernels read the rotated rows
    uint16_t* rq = reinterpret_cast<uint16_t*>(ws + gdn_ws_T(L) + gdn_ws_g(L) + gdn_ws_stage(L) + gdn_ws_map(L));
    const int64_t rows = int64_t(gdn_token_rows(L));
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
                  static_cast<const uint16_t*>(L.v), L.alpha, L.beta, L.buf_k, L.buf_v,
                  gdn_fp8_scales(L, L.buf_k), gdn_fp8_scales(L, L.buf_v), gdn_buf_fmt(L), L.buf_alpha,
                  L.buf_beta, sk, sq, sv, sa, sb, sm, L.B, L.H, L.buf_W, L.buf_d};
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
  // chunks per window (0: never requantized); windows of one chunk take the
  // kernel that keeps no fp32 state between chunks
  const int cpw = L.no_requant ? 0 : L.W / PC;
  StateArgs s{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k),
              static_cast<const uint16_t*>(L.v), L.beta, T_ws, g_ws, L.init_codes, L.init_scales,
              L.o, L.codes, L.scales, sm, L.B, L.H, cpw, L.no_requant ? L.state_f32 : nullptr};
  const unsigned grid = unsigned(L.B) * L.H * (PD / RWS);
  auto kern = cpw == 1
                  ? (L.q4 ? (L.out_bf16 ? &gdn_state_kernel<true, 4, false> : &gdn_state_kernel<false, 4, false>)
                          : (L.out_bf16 ? &gdn_state_kernel<true, 8, false> : &gdn_state_kernel<false, 8, false>))
                  : (L.q4 ? (L.out_bf16 ? &gdn_state_kernel<true, 4, true> : &gdn_state_kernel<false, 4, true>)
                          : (L.out_bf16 ? &gdn_state_kernel<true, 8, true> : &gdn_state_kernel<false, 8, true>));
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, STATE_LDS))
    return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(SNT), STATE_LDS, stream, s);
  if (hipError_t e = hipGetLastError()) return e;
  if (L.handoff && L.B > 0) {
    HandoffArgs h{static_cast<const uint16_t*>(L.k), static_cast<const uint16_t*>(L.v), L.alpha, L.beta,
                  L.buf_k, L.buf_v, gdn_fp8_scales(L, L.buf_k), gdn_fp8_scales(L, L.buf_v), gdn_buf_fmt(L),
                  L.buf_alpha, L.buf_beta, L.fill_out, sm, L.B, L.H, L.buf_W, L.buf_d};
    hipLaunchKernelGGL(gdn_handoff_kernel, dim3(unsigned(L.B) * L.H), dim3(256), 0, stream, h);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdnq
