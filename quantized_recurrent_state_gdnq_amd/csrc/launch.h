// Internal launch interface between the C ABI (abi.cpp) and the kernels.
// Shapes are validated by the ABI before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdnq {

struct QuantizeLaunch {
  const float* S;
  int64_t rows;
  int d_k;
  int8_t* codes;
  float* scales;
  bool wht;
  bool q4;  // 4-bit codes, two per byte
};
hipError_t launch_quantize(const QuantizeLaunch& L, hipStream_t stream);

struct DecodeLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  int8_t* codes;
  float* scales;
  void* buf_k;    // fp32, bf16 with buf_bf16, or E4M3 codes + per-vector scales with buf_fp8
  void* buf_v;
  float* buf_alpha;
  float* buf_beta;
  const int32_t* fill_in;
  int32_t* fill_out;
  void* o;
  int B, H, d_k, d_v, W;
  bool in_bf16, out_bf16, wht, buf_bf16, buf_fp8;
  bool q4;  // 4-bit state codes, two per byte
  bool sliding;  // the Pure-Write sliding window (ring buffer, requantize every token)
};
hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);
hipError_t launch_decode_sliding(const DecodeLaunch& L, hipStream_t stream);
int decode_row_split();
int decode_max_batch();
void set_decode_schedule(int grid, int open_waves);  // 0 = default

struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const int8_t* init_codes;
  const float* init_scales;
  void* o;
  int8_t* codes;
  float* scales;
  float* state_f32;
  void* workspace;
  void* buf_k;  // hand-over to decode (GDN): the open window's writes and the fill
  void* buf_v;   // (fp32, bf16 or FP8 vector pairs as decode keeps them)
  float* buf_alpha;
  float* buf_beta;
  int32_t* fill_out;
  const int32_t* cu_seqlens;  // variable lengths (GDN hand-over): B + 1 token offsets on the device, T their total
  const int32_t* fill_in;     // resuming (GDN hand-over): writes each sequence's window buffer holds
  int B, T, H, d_k, d_v, C, W;
  bool out_bf16, wht, ssd, int8_qk, handoff, varlen, resume;
  bool q4;  // GDN: the state as packed 4-bit codes
  bool buf_bf16, buf_fp8;  // hand-over: the window buffer's format
  bool no_requant;  // GDN: never requantize; the final fp32 state goes to state_f32
  int buf_W, buf_d;  // hand-over: decode's window (slots per head) and vector length of its buffer
};
hipError_t launch_prefill_gdn(const PrefillLaunch& L, hipStream_t stream);
hipError_t launch_prefill_ssd(const PrefillLaunch& L, hipStream_t stream);
size_t prefill_gdn_workspace_bytes(const PrefillLaunch& L);
size_t prefill_ssd_workspace_bytes(const PrefillLaunch& L);
// Device scratch of the allocation-free prefill (scratch.hip): its size, and
// its address on the current device (looked up once per device).
size_t scratch_capacity();
hipError_t scratch_for_current_device(void** out);

inline size_t prefill_workspace_bytes(const PrefillLaunch& L) {
  return L.ssd ? prefill_ssd_workspace_bytes(L) : prefill_gdn_workspace_bytes(L);
}

}  // namespace gdnq
