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
// (codes * row scale) and S_C is requantized at every chunk end.
//
// Two kernels:
//   prep  -- one workgroup per chunk-head, all in parallel: K K^T on bf16
//            MFMA (bf16 inputs, exact products), A, and T by blocked forward
//            substitution in fp32; T and g go to the workspace.
//   state -- one workgroup per (sequence, head, block of 32 rows): rows of
//            the state evolve independently, so each workgroup carries its
//            rows (int8 codes + scales in LDS) through all chunks.  K S0^T and
//            Q S0^T use exact bf16 products with the int8 codes; the state
//            update multiplies an fp32 operand split into three bf16 parts
//            (24 significant bits) by exact bf16 keys.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "mfma.h"

namespace gdnq {

constexpr int PC = 64;    // chunk = window
constexpr int PD = 128;   // d_k = d_v
constexpr int KP = 136;   // LDS pitch (bf16) of [token][dim] tiles (padding spreads banks)
constexpr int KTP = 72;   // LDS pitch (bf16) of [dim][token]
constexpr int AP = 65;    // LDS pitch (fp32) of A in the prep kernel
constexpr int RWS = 32;   // state rows per workgroup
constexpr int CP = 144;   // LDS pitch (bytes) of the int8 rows
constexpr int UTP = 68;   // LDS pitch (fp32) of U^T
constexpr int SP = 132;   // LDS pitch (fp32) of the new state rows

__device__ __forceinline__ void tile_of(int tt, int& it, int& jt) {
  it = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;  // lower tiles (it >= jt), row-major
  jt = tt - it * (it + 1) / 2;
}

struct PrepArgs {
  const uint16_t* k;
  const float* alpha;
  const float* beta;
  float* T_ws;  // [B*NC*H][64][64]
  float* g_ws;  // [B*NC*H][64]
  int B, T, H;
};

__global__ __launch_bounds__(256) void gdn_prep_kernel(PrepArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 Kl[PC * KP];
  __shared__ float Al[PC * AP];
  __shared__ __attribute__((aligned(16))) float Tl[PC * PC];
  __shared__ float Pl[3 * 256];
  __shared__ float gl[PC], bl[PC];
  const int NC = a.T / PC;
  const int idx = blockIdx.x;  // (b * NC + c) * H + h
  const int h = idx % a.H;
  const int c = (idx / a.H) % NC;
  const int b = idx / (a.H * NC);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t tok0 = size_t(b) * a.T + size_t(c) * PC;

  {  // keys of the chunk: thread -> token tid / 4, dims [(tid % 4) * 32, +32)
    const int i = tid >> 2, qq = tid & 3;
    const uint4* src = reinterpret_cast<const uint4*>(a.k + ((tok0 + i) * a.H + h) * PD + qq * 32);
    uint4 w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = src[e];
    uint4* dst = reinterpret_cast<uint4*>(Kl + i * KP + qq * 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = w[e];
  }
  if (tid < 64) {  // g = inclusive prefix sum of log alpha
    const size_t r = (tok0 + tid) * a.H + h;
    float la = logf(a.alpha[r]);
    bl[tid] = a.beta[r];
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const float o = __shfl_up(la, s, 64);
      if (lane >= s) la += o;
    }
    gl[tid] = la;
    a.g_ws[size_t(idx) * PC + tid] = la;
  }
  for (int e = tid; e < PC * PC; e += 256) Tl[e] = 0.f;
  __syncthreads();

  // A from the lower 16x16 tiles of K K^T
  for (int tt = wave; tt < 10; tt += 4) {
    int it, jt;
    tile_of(tt, it, jt);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = ks * 32 + 8 * (lane >> 4);
      acc = mfma16(lds_bf16x8(Kl + (it * 16 + (lane & 15)) * KP + kk),
                   lds_bf16x8(Kl + (jt * 16 + (lane & 15)) * KP + kk), acc);
    }
    const int j = jt * 16 + (lane & 15);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = it * 16 + 4 * (lane >> 4) + q;
      Al[i * AP + j] = (j < i) ? bl[i] * expf(gl[i] - gl[j]) * acc[q] : 0.f;
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
      for (int j = 0; j < r; ++j) s -= Al[(bb * 16 + r) * AP + bb * 16 + j] * t[j];
      t[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tl[(bb * 16 + r) * PC + bb * 16 + cc] = t[r];
  }
  __syncthreads();

  // off-diagonal blocks, one block-diagonal at a time:
  //   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  for (int d = 1; d <= 3; ++d) {
    const int nb = 4 - d;
    const int r = tid >> 4, cc = tid & 15;
    for (int m = 0; m < nb; ++m) {
      const int i = d + m, j = m;
      float s = 0.f;
      for (int kb = j; kb < i; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) s += Al[(i * 16 + r) * AP + kb * 16 + x] * Tl[(kb * 16 + x) * PC + j * 16 + cc];
      Pl[m * 256 + r * 16 + cc] = s;
    }
    __syncthreads();
    for (int m = 0; m < nb; ++m) {
      const int i = d + m, j = m;
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) s += Tl[(i * 16 + r) * PC + i * 16 + x] * Pl[m * 256 + x * 16 + cc];
      Tl[(i * 16 + r) * PC + j * 16 + cc] = -s;
    }
    __syncthreads();
  }

  float4* dst = reinterpret_cast<float4*>(a.T_ws + size_t(idx) * PC * PC);
  for (int e = tid; e < PC * PC / 4; e += 256) dst[e] = reinterpret_cast<const float4*>(Tl)[e];
}

struct StateArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* beta;
  const float* T_ws;
  const float* g_ws;
  const int8_t* init_codes;
  const float* init_scales;
  void* o;
  int8_t* codes;
  float* scales;
  int B, T, H;
};

template <bool OUT_BF16>
__global__ __launch_bounds__(512) void gdn_state_kernel(StateArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __bf16* Kl = reinterpret_cast<__bf16*>(lds);                       // [64][KP]
  __bf16* KTl = Kl + PC * KP;                                         // [128][KTP]
  __bf16* Ql = KTl + PD * KTP;                                        // [64][KP]
  __bf16* Vl = Ql + PC * KP;                                          // [64][32]
  float* Tl = reinterpret_cast<float*>(Vl + PC * RWS);                // [64][64]
  float* Rl = Tl + PC * PC;                                           // [64][32] rhs
  float* Ul = Rl + PC * RWS;                                          // [64][32]
  float* UTl = Ul + PC * RWS;                                         // [32][UTP]
  float* OSl = UTl + RWS * UTP;                                       // [64][32]
  float* Ml = OSl + PC * RWS;                                         // [64][64], then new rows [32][SP]
  float* gl = Ml + RWS * SP;                                          // [64] g
  float* el = gl + PC;                                                // [64] exp(g)
  float* dl = el + PC;                                                // [64] exp(g_C - g)
  float* bl = dl + PC;                                                // [64] beta
  float* sl = bl + PC;                                                // [32] row scales
  int8_t* cl = reinterpret_cast<int8_t*>(sl + RWS);                   // [32][CP] int8 rows

  const int nblk = a.B * a.H * (PD / RWS);
  const int logical = xcd_swizzle(blockIdx.x, nblk);  // the 4 row blocks of a head share an XCD
  const int chain = logical / (PD / RWS);
  const int rb = logical % (PD / RWS);
  const int b = chain / a.H, h = chain % a.H;
  const int r0 = rb * RWS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NC = a.T / PC;
  const size_t state_row0 = (size_t(b) * a.H + h) * PD + r0;

  // stored rows at the start (zero state without init)
  {
    const int r = tid >> 4, seg = tid & 15;  // 32 rows x 16 segments of 8 codes
    uint2 w = make_uint2(0u, 0u);
    if (a.init_codes) w = *reinterpret_cast<const uint2*>(a.init_codes + (state_row0 + r) * PD + seg * 8);
    *reinterpret_cast<uint2*>(cl + r * CP + seg * 8) = w;
    if (seg == 0) sl[r] = a.init_scales ? a.init_scales[state_row0 + r] : 0.f;
  }

  for (int c = 0; c < NC; ++c) {
    const size_t tok0 = size_t(b) * a.T + size_t(c) * PC;
    const size_t ch = (size_t(b) * NC + c) * a.H + h;
    __syncthreads();  // previous chunk done with every buffer
    {  // K (row-major and transposed) and Q: thread -> token tid / 8, dims [(tid % 8) * 16, +16)
      const int i = tid >> 3, s8 = tid & 7;
      const uint4* ks = reinterpret_cast<const uint4*>(a.k + ((tok0 + i) * a.H + h) * PD + s8 * 16);
      const uint4* qs = reinterpret_cast<const uint4*>(a.q + ((tok0 + i) * a.H + h) * PD + s8 * 16);
      const uint4 k0 = ks[0], k1 = ks[1], q0 = qs[0], q1 = qs[1];
      uint4* kd = reinterpret_cast<uint4*>(Kl + i * KP + s8 * 16);
      kd[0] = k0;
      kd[1] = k1;
      uint4* qd = reinterpret_cast<uint4*>(Ql + i * KP + s8 * 16);
      qd[0] = q0;
      qd[1] = q1;
      const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      uint16_t* kt = reinterpret_cast<uint16_t*>(KTl);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kt[(s8 * 16 + 2 * e) * KTP + i] = uint16_t(kw[e] & 0xffffu);
        kt[(s8 * 16 + 2 * e + 1) * KTP + i] = uint16_t(kw[e] >> 16);
      }
    }
    if (tid < 256) {  // this workgroup's rows of V: token tid / 4, rows [(tid % 4) * 8, +8)
      const int i = tid >> 2, q4 = tid & 3;
      *reinterpret_cast<uint4*>(Vl + i * RWS + q4 * 8) =
          *reinterpret_cast<const uint4*>(a.v + ((tok0 + i) * a.H + h) * PD + r0 + q4 * 8);
    }
    {  // T of the chunk
      const float4* ts = reinterpret_cast<const float4*>(a.T_ws + ch * PC * PC);
      float4* td = reinterpret_cast<float4*>(Tl);
      td[tid] = ts[tid];
      td[tid + 512] = ts[tid + 512];
    }
    if (tid < 64) {
      const float g = a.g_ws[ch * PC + tid];
      gl[tid] = g;
      el[tid] = expf(g);
      bl[tid] = a.beta[(tok0 + tid) * a.H + h];
    }
    __syncthreads();
    if (tid < 64) dl[tid] = expf(gl[PC - 1] - gl[tid]);

    {  // X = K S0^T and Q S0^T for token tile it, row tile rt; then rhs and the output base
      const int it = wave >> 1, rt = wave & 1;
      f32x4 xacc = {0.f, 0.f, 0.f, 0.f}, qacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * (lane >> 4);
        const bf16x8 bc = i8x8_to_bf16(*reinterpret_cast<const uint2*>(cl + (rt * 16 + (lane & 15)) * CP + kk));
        xacc = mfma16(lds_bf16x8(Kl + (it * 16 + (lane & 15)) * KP + kk), bc, xacc);
        qacc = mfma16(lds_bf16x8(Ql + (it * 16 + (lane & 15)) * KP + kk), bc, qacc);
      }
      const int r = rt * 16 + (lane & 15);
      const float sr = sl[r];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = it * 16 + 4 * (lane >> 4) + q;
        const float gi = el[i];
        Rl[i * RWS + r] = bl[i] * (float(Vl[i * RWS + r]) - gi * (sr * xacc[q]));
        OSl[i * RWS + r] = gi * (sr * qacc[q]);
      }
    }
    __syncthreads();

    {  // U = T rhs (T unit lower triangular)
      const int r = tid & 31, ib = tid >> 5;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int i = ib + 16 * qq;
        float s = 0.f;
        for (int j = 0; j <= i; ++j) s += Tl[i * PC + j] * Rl[j * RWS + r];
        Ul[i * RWS + r] = s;
        UTl[r * UTP + i] = s;
      }
    }
    // M = L o Q K^T on the lower tiles (upper tiles are never read)
    for (int tt = wave; tt < 10; tt += 8) {
      int it, jt;
      tile_of(tt, it, jt);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kk = ks * 32 + 8 * (lane >> 4);
        acc = mfma16(lds_bf16x8(Ql + (it * 16 + (lane & 15)) * KP + kk),
                     lds_bf16x8(Kl + (jt * 16 + (lane & 15)) * KP + kk), acc);
      }
      const int j = jt * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = it * 16 + 4 * (lane >> 4) + q;
        Ml[i * PC + j] = (j <= i) ? expf(gl[i] - gl[j]) * acc[q] : 0.f;
      }
    }
    __syncthreads();

    {  // O = O_base + M U
      const int r = tid & 31, ib = tid >> 5;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int i = ib + 16 * qq;
        float s = OSl[i * RWS + r];
        for (int j = 0; j <= i; ++j) s += Ml[i * PC + j] * Ul[j * RWS + r];
        const size_t oi = ((tok0 + i) * a.H + h) * PD + r0 + r;
        if constexpr (OUT_BF16) static_cast<uint16_t*>(a.o)[oi] = uint16_t(f32_to_bf16_bits(s));
        else static_cast<float*>(a.o)[oi] = s;
      }
    }
    __syncthreads();  // M is overwritten by the new rows below

    {  // S_C = gamma_C S0 + (U o d)^T K: row tile rt, column tiles ct0, ct0 + 1
      const int rt = wave >> 2, ct0 = (wave & 3) * 2;
      const int r = rt * 16 + (lane & 15);
      bf16x8 a1[2], a2[2], a3[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kk = ks * 32 + 8 * (lane >> 4);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = UTl[r * UTP + kk + e] * dl[kk + e];
        split3(x, a1[ks], a2[ks], a3[ks]);
      }
      const float gC = el[PC - 1];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ct = ct0 + cc;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 bk = lds_bf16x8(KTl + (ct * 16 + (lane & 15)) * KTP + ks * 32 + 8 * (lane >> 4));
          acc = mfma16(a1[ks], bk, acc);
          acc = mfma16(a2[ks], bk, acc);
          acc = mfma16(a3[ks], bk, acc);
        }
        const int col = ct * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = rt * 16 + 4 * (lane >> 4) + q;
          const float s0 = float(cl[rr * CP + col]) * sl[rr];
          Ml[rr * SP + col] = gC * s0 + acc[q];
        }
      }
    }
    __syncthreads();

    {  // requantize the new rows: row tid / 16, columns [(tid % 16) * 8, +8)
      const int r = tid >> 4, seg = tid & 15;
      float x[8];
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = Ml[r * SP + seg * 8 + e];
        amax = fmaxf(amax, fabsf(x[e]));
      }
      amax = group_max<16>(amax);
      const float scale = codec_scale(amax);
      uint2 w;
      w.x = pack4_i8(codec_code(x[0], scale), codec_code(x[1], scale), codec_code(x[2], scale), codec_code(x[3], scale));
      w.y = pack4_i8(codec_code(x[4], scale), codec_code(x[5], scale), codec_code(x[6], scale), codec_code(x[7], scale));
      *reinterpret_cast<uint2*>(cl + r * CP + seg * 8) = w;
      if (seg == 0) sl[r] = scale;
    }
  }
  __syncthreads();
  {  // final rows
    const int r = tid >> 4, seg = tid & 15;
    *reinterpret_cast<uint2*>(a.codes + (state_row0 + r) * PD + seg * 8) =
        *reinterpret_cast<const uint2*>(cl + r * CP + seg * 8);
    if (seg == 0) a.scales[state_row0 + r] = sl[r];
  }
}

static size_t state_lds_bytes() {
  return size_t(PC * KP + PD * KTP + PC * KP + PC * RWS) * 2 +
         size_t(PC * PC + 3 * PC * RWS + RWS * UTP + PC * RWS + RWS * SP + 4 * PC + RWS) * 4 +
         size_t(RWS * CP);
}

static size_t gdn_ws_T(const PrefillLaunch& L) { return size_t(L.B) * (L.T / PC) * L.H * PC * PC * 4; }
static size_t gdn_ws_g(const PrefillLaunch& L) { return size_t(L.B) * (L.T / PC) * L.H * PC * 4; }

size_t prefill_gdn_workspace_bytes(const PrefillLaunch& L) { return gdn_ws_T(L) + gdn_ws_g(L); }

hipError_t launch_prefill_gdn(const PrefillLaunch& L, hipStream_t stream) {
  float* T_ws = static_cast<float*>(L.workspace);
  float* g_ws = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + gdn_ws_T(L));
  const int NC = L.T / PC;
  if (NC > 0) {
    PrepArgs p{static_cast<const uint16_t*>(L.k), L.alpha, L.beta, T_ws, g_ws, L.B, L.T, L.H};
    hipLaunchKernelGGL(gdn_prep_kernel, dim3(unsigned(L.B) * NC * L.H), dim3(256), 0, stream, p);
    if (hipError_t e = hipGetLastError()) return e;
  }
  StateArgs s{static_cast<const uint16_t*>(L.q), static_cast<const uint16_t*>(L.k),
              static_cast<const uint16_t*>(L.v), L.beta, T_ws, g_ws, L.init_codes, L.init_scales,
              L.o, L.codes, L.scales, L.B, L.T, L.H};
  const size_t lds = state_lds_bytes();
  const unsigned grid = unsigned(L.B) * L.H * (PD / RWS);
  if (L.out_bf16) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_state_kernel<true>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    hipLaunchKernelGGL(gdn_state_kernel<true>, dim3(grid), dim3(512), lds, stream, s);
  } else {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_state_kernel<false>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    hipLaunchKernelGGL(gdn_state_kernel<false>, dim3(grid), dim3(512), lds, stream, s);
  }
  return hipGetLastError();
}

}  // namespace gdnq
