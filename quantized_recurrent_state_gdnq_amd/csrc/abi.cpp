// C ABI of the library: argument validation, error reporting and dispatch to
// the gfx950 kernels.  Validation is complete before anything is launched;
// on any error nothing is launched and nothing is written.
#include "../../include/gdnq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

gdnq_status fail(gdnq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gdnq_status ok() {
  g_err[0] = '\0';
  return GDNQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const char* name;
  const void* p;
  size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

gdnq_status check_ptrs(const Span* s, int n) {
  for (int i = 0; i < n; ++i)
    if (!s[i].p) return fail(GDNQ_ERR_NULL, "%s is NULL", s[i].name);
  for (int i = 0; i < n; ++i)
    if (!aligned16(s[i].p)) return fail(GDNQ_ERR_ALIGN, "%s is not 16-byte aligned", s[i].name);
  return GDNQ_OK;
}

// HIP keeps the last error of any runtime call per thread until it is read;
// clear it before a launch so that the status reported is the launch's own.
void clear_stale_hip_error() { (void)hipGetLastError(); }

gdnq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDNQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// GDNQ_SYNC_DEBUG=1 in the environment when the library is loaded: every call
// waits for its kernels on its stream and reports a fault of theirs as its own
// GDNQ_ERR_HIP, naming the call, instead of leaving it to the caller's next
// synchronization.  Read once; the default is fully asynchronous.
const bool g_sync_debug = [] {
  const char* e = std::getenv("GDNQ_SYNC_DEBUG");
  return e && e[0] == '1' && e[1] == '\0';
}();

gdnq_status launched(hipError_t e, const char* what, void* stream) {
  if (e == hipSuccess && g_sync_debug) {
    e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(GDNQ_ERR_HIP, "%s (synchronized under GDNQ_SYNC_DEBUG): %s", what, hipGetErrorString(e));
  }
  return hip_status(e, what);
}

bool dim_ok(int d) { return d == 64 || d == 128; }
size_t esize(int32_t dt) { return dt == GDNQ_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char* gdnq_status_string(gdnq_status s) {
  switch (s) {
    case GDNQ_OK: return "ok";
    case GDNQ_ERR_NULL: return "null pointer";
    case GDNQ_ERR_SHAPE: return "unsupported shape";
    case GDNQ_ERR_DTYPE: return "unsupported dtype";
    case GDNQ_ERR_ALIGN: return "misaligned pointer";
    case GDNQ_ERR_ALIAS: return "aliased buffers";
    case GDNQ_ERR_WORKSPACE: return "workspace too small";
    case GDNQ_ERR_HIP: return "HIP runtime error";
    case GDNQ_ERR_FLAGS: return "unsupported flags";
  }
  return "unknown status";
}

const char* gdnq_last_error(void) { return g_err; }

int32_t gdnq_version(void) { return 101; }

int32_t gdnq_sync_debug(void) { return g_sync_debug ? 1 : 0; }

gdnq_status gdnq_decode_set_schedule(int32_t grid, int32_t open_waves) {
  if (grid < 0 || open_waves < 0)
    return fail(GDNQ_ERR_SHAPE, "grid = %d, open_waves = %d: 0 (default) or positive", grid, open_waves);
  gdnq::set_decode_schedule(grid, open_waves);
  return ok();
}

gdnq_status gdnq_quantize_state(const float* S, int64_t rows, int32_t d_k, int8_t* codes,
                                float* scales, uint32_t flags, void* stream) {
  if (rows < 0) return fail(GDNQ_ERR_SHAPE, "rows = %lld < 0", (long long)rows);
  if (!dim_ok(d_k)) return fail(GDNQ_ERR_SHAPE, "d_k = %d, expected 64 or 128", d_k);
  if (flags & ~uint32_t(GDNQ_FLAG_WHT | GDNQ_FLAG_STATE_4BIT))
    return fail(GDNQ_ERR_FLAGS, "flags 0x%x: only GDNQ_FLAG_WHT and GDNQ_FLAG_STATE_4BIT allowed", flags);
  const bool q4 = (flags & GDNQ_FLAG_STATE_4BIT) != 0;
  if (rows > (int64_t(1) << 35)) return fail(GDNQ_ERR_SHAPE, "rows = %lld too large", (long long)rows);
  if (rows == 0) return ok();
  const Span sp[] = {{"S", S, size_t(rows) * d_k * 4}, {"codes", codes, size_t(rows) * d_k / (q4 ? 2 : 1)},
                     {"scales", scales, size_t(rows) * 4}};
  if (gdnq_status st = check_ptrs(sp, 3)) return st;
  if (overlap(sp[0], sp[1]) || overlap(sp[0], sp[2]) || overlap(sp[1], sp[2]))
    return fail(GDNQ_ERR_ALIAS, "S, codes and scales must not overlap");
  clear_stale_hip_error();
  gdnq::QuantizeLaunch L{S, rows, d_k, codes, scales, (flags & GDNQ_FLAG_WHT) != 0, q4};
  return launched(gdnq::launch_quantize(L, static_cast<hipStream_t>(stream)), "quantize launch", stream);
}

gdnq_status gdnq_decode_step(const gdnq_decode_params* p, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta,
                             int8_t* codes, float* scales, void* buf_k, void* buf_v,
                             float* buf_alpha, float* buf_beta, const int32_t* fill_in,
                             int32_t* fill_out, void* o, void* stream) {
  if (!p) return fail(GDNQ_ERR_NULL, "params is NULL");
  const int B = p->batch, H = p->heads, dk = p->d_k, dv = p->d_v, W = p->window;
  if (B < 0) return fail(GDNQ_ERR_SHAPE, "batch = %d < 0", B);
  if (H < 1) return fail(GDNQ_ERR_SHAPE, "heads = %d < 1", H);
  if (!dim_ok(dk) || !dim_ok(dv)) return fail(GDNQ_ERR_SHAPE, "d_k = %d, d_v = %d: each must be 64 or 128", dk, dv);
  if (W < 1 || W > 64) return fail(GDNQ_ERR_SHAPE, "window = %d, expected 1..64", W);
  if ((p->in_dtype != GDNQ_F32 && p->in_dtype != GDNQ_BF16) ||
      (p->out_dtype != GDNQ_F32 && p->out_dtype != GDNQ_BF16))
    return fail(GDNQ_ERR_DTYPE, "in_dtype = %d, out_dtype = %d", p->in_dtype, p->out_dtype);
  if (p->flags & ~uint32_t(GDNQ_FLAG_WHT | GDNQ_FLAG_BUF_BF16 | GDNQ_FLAG_BUF_FP8 | GDNQ_FLAG_STATE_4BIT |
                           GDNQ_FLAG_SLIDING))
    return fail(GDNQ_ERR_FLAGS,
                "flags 0x%x: decode accepts GDNQ_FLAG_WHT, GDNQ_FLAG_BUF_BF16, GDNQ_FLAG_BUF_FP8, "
                "GDNQ_FLAG_STATE_4BIT, GDNQ_FLAG_SLIDING",
                p->flags);
  const bool sliding = (p->flags & GDNQ_FLAG_SLIDING) != 0;
  if (sliding && (p->flags & (GDNQ_FLAG_BUF_BF16 | GDNQ_FLAG_BUF_FP8 | GDNQ_FLAG_STATE_4BIT)))
    return fail(GDNQ_ERR_FLAGS, "flags 0x%x: GDNQ_FLAG_SLIDING keeps an fp32 window and an 8-bit state", p->flags);
  const bool q4 = (p->flags & GDNQ_FLAG_STATE_4BIT) != 0;
  const bool buf_bf16 = (p->flags & GDNQ_FLAG_BUF_BF16) != 0;
  const bool buf_fp8 = (p->flags & GDNQ_FLAG_BUF_FP8) != 0;
  if (buf_bf16 && buf_fp8)
    return fail(GDNQ_ERR_FLAGS, "flags 0x%x: GDNQ_FLAG_BUF_BF16 and GDNQ_FLAG_BUF_FP8 are exclusive", p->flags);
  if (B > gdnq::decode_max_batch())
    return fail(GDNQ_ERR_SHAPE, "batch = %d, at most %d sequences per call", B, gdnq::decode_max_batch());
  if (int64_t(B) * H * gdnq::decode_row_split() > 0x7fffffffLL)
    return fail(GDNQ_ERR_SHAPE, "batch * heads = %lld too large", (long long)B * H);
  if (B == 0) return ok();
  const size_t bh = size_t(B) * H, ei = esize(p->in_dtype), eo = esize(p->out_dtype);
  const Span sp[] = {{"q", q, bh * dk * ei},
                     {"k", k, bh * dk * ei},
                     {"v", v, bh * dv * ei},
                     {"alpha", alpha, bh * 4},
                     {"beta", beta, bh * 4},
                     {"codes", codes, bh * dv * dk / (q4 ? 2 : 1)},
                     {"scales", scales, bh * dv * 4},
                     {"buf_k", buf_k, bh * W * (buf_fp8 ? dk + 4 : dk * (buf_bf16 ? 2 : 4))},
                     {"buf_v", buf_v, bh * W * (buf_fp8 ? dv + 4 : dv * (buf_bf16 ? 2 : 4))},
                     {"buf_alpha", buf_alpha, bh * W * 4},
                     {"buf_beta", buf_beta, bh * W * 4},
                     {"fill_in", fill_in, size_t(B) * 4},
                     {"fill_out", fill_out, size_t(B) * 4},
                     {"o", o, bh * dv * eo}};
  constexpr int N = sizeof(sp) / sizeof(sp[0]);
  if (gdnq_status st = check_ptrs(sp, N)) return st;
  // every written buffer (codes .. fill_out, o) must be disjoint from every other buffer
  for (int i = 5; i < N; ++i) {
    if (i == 11) continue;  // fill_in is read-only
    for (int j = 0; j < N; ++j)
      if (j != i && overlap(sp[i], sp[j]))
        return fail(GDNQ_ERR_ALIAS, "%s overlaps %s", sp[i].name, sp[j].name);
  }
  clear_stale_hip_error();
  gdnq::DecodeLaunch L{q,        k,        v,       alpha, beta, codes, scales, buf_k,
                       buf_v,    buf_alpha, buf_beta, fill_in, fill_out, o,   B,      H,
                       dk,       dv,       W,       p->in_dtype == GDNQ_BF16,
                       p->out_dtype == GDNQ_BF16, (p->flags & GDNQ_FLAG_WHT) != 0, buf_bf16, buf_fp8, q4,
                       sliding};
  return launched(gdnq::launch_decode(L, static_cast<hipStream_t>(stream)), "decode launch", stream);
}

// What the prefill entry points take: chunked (whole windows; any window),
// the uniform hand-over to decode (any T; decode's window 1 .. 64), and the
// variable-length and resuming hand-overs (packed or per-sequence lengths,
// decode's window 1 .. 64).
enum PrefillMode { PF_CHUNKED = 0, PF_HANDOFF = 1, PF_MAPPED = 2 };

static gdnq_status prefill_validate(const gdnq_prefill_params* p, gdnq::PrefillLaunch& L, int mode = PF_CHUNKED) {
  const bool handoff = mode != PF_CHUNKED, mapped = mode == PF_MAPPED;
  if (!p) return fail(GDNQ_ERR_NULL, "params is NULL");
  const int B = p->batch, T = p->seqlen, H = p->heads, dk = p->d_k, dv = p->d_v;
  if (B < 0 || T < 0 || H < 1) return fail(GDNQ_ERR_SHAPE, "batch = %d, seqlen = %d, heads = %d", B, T, H);
  if (p->in_dtype != GDNQ_BF16) return fail(GDNQ_ERR_DTYPE, "prefill in_dtype must be GDNQ_BF16");
  if (p->out_dtype != GDNQ_F32 && p->out_dtype != GDNQ_BF16) return fail(GDNQ_ERR_DTYPE, "out_dtype = %d", p->out_dtype);
  const bool ssd = (p->flags & GDNQ_FLAG_SSD) != 0;
  const bool no_rq = (p->flags & GDNQ_FLAG_NO_REQUANT) != 0;
  const int C = p->chunk, W = p->window;
  // GDN: chunk in {16, 32, 64} and any window (the kernels run every window
  // as whole 64-position chunks, so the result depends on the window only and
  // the chunk is a blocking hint); the hand-over calls take decode's windows
  // (1 .. 64); SSD takes chunk = 64
  if (ssd) {
    if (C != 64) return fail(GDNQ_ERR_SHAPE, "chunk = %d, expected 64", C);
  } else {
    if (C != 16 && C != 32 && C != 64) return fail(GDNQ_ERR_SHAPE, "chunk = %d, expected 16, 32 or 64", C);
    const int wmax = handoff ? 64 : GDNQ_MAX_WINDOW;
    if (W < 1 || W > wmax) return fail(GDNQ_ERR_SHAPE, "window = %d, expected 1 .. %d", W, wmax);
  }
  if (no_rq && (ssd || handoff))
    return fail(GDNQ_ERR_FLAGS, "GDNQ_FLAG_NO_REQUANT: GDN gdnq_prefill_chunked only");
  // whole windows (the SSD recurrence has none: whole chunks; a state that
  // is never requantized has none either: any length)
  const int Wt = ssd ? 64 : no_rq ? 1 : W;
  if (T % Wt && !handoff) return fail(GDNQ_ERR_SHAPE, "seqlen = %d is not a multiple of the window (%d)", T, Wt);
  // positions the chunk kernels see: windows padded to whole 64-position
  // chunks (the hand-over's open last window unpadded)
  const bool padded_map = mapped && (W < 64 || dk == 64);  // a sequence's padded length <= 64 (T + W - 1) / W
  const int64_t Tk = ssd        ? int64_t(T)
                     : no_rq      ? (int64_t(T) + 63) / 64 * 64
                     : padded_map ? (64 * (int64_t(T) + W - 1) + W - 1) / W
                                  : int64_t(T) / W * ((int64_t(W) + 63) / 64 * 64) + T % W;
  if ((Tk + 64) * H * 512 >= (int64_t(1) << 32))  // 32-bit output offsets, padding positions included
    return fail(GDNQ_ERR_SHAPE, "seqlen * heads = %lld: one sequence's outputs must stay under 4 GiB",
                (long long)T * H);
  if (ssd && handoff) return fail(GDNQ_ERR_FLAGS, "the hand-over to decode is for the GDN recurrence (no GDNQ_FLAG_SSD)");
  if (ssd) {
    if (p->flags & ~uint32_t(GDNQ_FLAG_SSD | GDNQ_FLAG_WHT | GDNQ_FLAG_INT8_QK))
      return fail(GDNQ_ERR_FLAGS, "flags 0x%x", p->flags);
    if (!dim_ok(dk) || !dim_ok(dv)) return fail(GDNQ_ERR_SHAPE, "SSD: d_k = %d, d_v = %d: each must be 64 or 128", dk, dv);
  } else {
    const uint32_t bufs = GDNQ_FLAG_BUF_BF16 | GDNQ_FLAG_BUF_FP8;
    if (p->flags & ~uint32_t(GDNQ_FLAG_STATE_4BIT | GDNQ_FLAG_WHT | GDNQ_FLAG_NO_REQUANT | (handoff ? bufs : 0u)))
      return fail(GDNQ_ERR_FLAGS, "flags 0x%x: GDN prefill takes GDNQ_FLAG_STATE_4BIT, GDNQ_FLAG_WHT and "
                  "GDNQ_FLAG_NO_REQUANT (the hand-over, varlen and resume calls GDNQ_FLAG_STATE_4BIT and one "
                  "window-buffer format flag)", p->flags);
    if ((p->flags & bufs) == bufs)
      return fail(GDNQ_ERR_FLAGS, "GDNQ_FLAG_BUF_BF16 and GDNQ_FLAG_BUF_FP8 are exclusive");
    if (!((dk == 128 && dv == 128) || (dk == 64 && dv == 64)))
      return fail(GDNQ_ERR_SHAPE, "GDN prefill: d_k = d_v = 128 or 64 required (got %d, %d)", dk, dv);
    if (dk == 64 && (p->flags & GDNQ_FLAG_WHT))
      return fail(GDNQ_ERR_FLAGS, "GDN prefill at d = 64 takes no GDNQ_FLAG_WHT");
  }
  if (int64_t(B) * H * 8 > 0x7fffffffLL) return fail(GDNQ_ERR_SHAPE, "batch * heads too large");
  L = gdnq::PrefillLaunch{};
  L.B = B; L.T = T; L.H = H; L.d_k = dk; L.d_v = dv; L.C = p->chunk; L.W = p->window;
  L.out_bf16 = p->out_dtype == GDNQ_BF16;
  L.wht = (p->flags & GDNQ_FLAG_WHT) != 0;
  L.ssd = ssd;
  L.int8_qk = (p->flags & GDNQ_FLAG_INT8_QK) != 0;
  L.q4 = !ssd && (p->flags & GDNQ_FLAG_STATE_4BIT) != 0;
  L.handoff = handoff;
  L.buf_bf16 = handoff && (p->flags & GDNQ_FLAG_BUF_BF16) != 0;
  L.buf_fp8 = handoff && (p->flags & GDNQ_FLAG_BUF_FP8) != 0;
  L.no_requant = no_rq;
  L.buf_W = W;
  L.buf_d = dk;
  return GDNQ_OK;
}

// The window-buffer arguments of gdnq_prefill_chunked make it the hand-over
// (also when T is not a multiple of the window).
static bool prefill_tail(const gdnq_prefill_params* p, const void* buf_k, const void* buf_v, const float* buf_alpha,
                         const float* buf_beta, const int32_t* fill_out) {
  if (buf_k || buf_v || buf_alpha || buf_beta || fill_out) return true;
  // SSD and GDNQ_FLAG_NO_REQUANT have no windows
  if (!p || (p->flags & (GDNQ_FLAG_SSD | GDNQ_FLAG_NO_REQUANT))) return false;
  return p->window > 0 && p->seqlen >= 0 && p->seqlen % p->window != 0;
}

size_t gdnq_prefill_workspace_size(const gdnq_prefill_params* p) {
  gdnq::PrefillLaunch L, H;
  const bool whole = prefill_validate(p, L) == GDNQ_OK;
  const bool handoff = !(p && (p->flags & GDNQ_FLAG_SSD)) && prefill_validate(p, H, PF_HANDOFF) == GDNQ_OK;
  const size_t a = whole ? gdnq::prefill_workspace_bytes(L) : 0, b = handoff ? gdnq::prefill_workspace_bytes(H) : 0;
  return a > b ? a : b;
}

// gdnq_prefill_chunked and its allocation-free variant: with noalloc, the
// workspace is the current device's scratch array (checked against its size
// after every other argument, before the one HIP query of its address).
static gdnq_status prefill_handoff_impl(gdnq::PrefillLaunch& L, const int32_t* cu_seqlens,
                                        const int32_t* fill_in, const void* q, const void* k, const void* v, const float* alpha,
                                        const float* beta, const int8_t* init_codes, const float* init_scales,
                                        void* o, int8_t* codes, float* scales, void* buf_k, void* buf_v,
                                        float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                        void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false);

// noalloc: the workspace is the current device's scratch array, checked
// against its size after every other argument, before the one HIP query of
// its address
static gdnq_status noalloc_workspace(size_t need, void*& workspace, size_t& workspace_bytes) {
  if (need > gdnq::scratch_capacity())
    return fail(GDNQ_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace; the allocation-free entry point holds at most %zu "
                "(use gdnq_prefill_chunked with a workspace, or split the batch)",
                need, gdnq::scratch_capacity());
  workspace = nullptr;
  workspace_bytes = 0;
  if (need > 0) {
    clear_stale_hip_error();
    if (gdnq_status st = hip_status(gdnq::scratch_for_current_device(&workspace), "device scratch lookup")) return st;
    workspace_bytes = gdnq::scratch_capacity();
  }
  return GDNQ_OK;
}

static gdnq_status prefill_chunked_impl(const gdnq_prefill_params* p, const void* q, const void* k,
                                        const void* v, const float* alpha, const float* beta,
                                        const int8_t* init_codes, const float* init_scales, void* o,
                                        int8_t* codes, float* scales, float* state_f32,
                                        void* buf_k, void* buf_v, float* buf_alpha, float* buf_beta,
                                        int32_t* fill_out, void* workspace, size_t workspace_bytes, void* stream,
                                        bool noalloc) {
  gdnq::PrefillLaunch L;
  if (prefill_tail(p, buf_k, buf_v, buf_alpha, buf_beta, fill_out)) {  // the hand-over to decode
    if (gdnq_status st = prefill_validate(p, L, PF_HANDOFF)) return st;
    if (state_f32) return fail(GDNQ_ERR_SHAPE, "state_f32 must be NULL when the window buffer is given (the state goes to codes and scales)");
    return prefill_handoff_impl(L, nullptr, nullptr, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales,
                                buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream, noalloc);
  }
  if (gdnq_status st = prefill_validate(p, L)) return st;
  if (L.B == 0) return ok();
  const size_t bth = size_t(L.B) * L.T * L.H, bh = size_t(L.B) * L.H;
  const size_t eo = L.out_bf16 ? 2 : 4;
  if (L.ssd) {
    if (beta || init_codes || init_scales || codes || scales)
      return fail(GDNQ_ERR_SHAPE, "SSD prefill: beta, init_codes, init_scales, codes, scales must be NULL");
    const Span sp[] = {{"q", q, bth * L.d_k * 2}, {"k", k, bth * L.d_k * 2},
                       {"v", v, bth * L.d_v * 2}, {"alpha", alpha, bth * 4},
                       {"o", o, bth * L.d_v * eo}, {"state_f32", state_f32, bh * L.d_v * L.d_k * 4}};
    constexpr int N = sizeof(sp) / sizeof(sp[0]);
    if (L.T > 0) {
      if (gdnq_status st = check_ptrs(sp, N)) return st;
    } else {
      if (gdnq_status st = check_ptrs(sp + 5, 1)) return st;
    }
    for (int i = 4; i < N; ++i)
      for (int j = 0; j < N; ++j)
        if (j != i && overlap(sp[i], sp[j])) return fail(GDNQ_ERR_ALIAS, "%s overlaps %s", sp[i].name, sp[j].name);
  } else {
    if (L.no_requant) {
      if (codes || scales)
        return fail(GDNQ_ERR_SHAPE, "GDNQ_FLAG_NO_REQUANT: codes and scales must be NULL (the final state goes to state_f32)");
    } else if (state_f32) {
      return fail(GDNQ_ERR_SHAPE, "GDN prefill: state_f32 must be NULL (it takes the state only under GDNQ_FLAG_NO_REQUANT)");
    }
    if ((init_codes == nullptr) != (init_scales == nullptr))
      return fail(GDNQ_ERR_NULL, "init_codes and init_scales must be both NULL or both set");
    Span sp[] = {{"q", q, bth * L.d_k * 2},         {"k", k, bth * L.d_k * 2},
                 {"v", v, bth * L.d_v * 2},         {"alpha", alpha, bth * 4},
                 {"beta", beta, bth * 4},           {"o", o, bth * L.d_v * eo},
                 {"codes", codes, bh * L.d_v * L.d_k / (L.q4 ? 2 : 1)}, {"scales", scales, bh * L.d_v * 4}};
    int N = sizeof(sp) / sizeof(sp[0]);
    if (L.no_requant) {  // the one state output
      sp[6] = {"state_f32", state_f32, bh * L.d_v * L.d_k * 4};
      N = 7;
    }
    if (L.T > 0) {
      if (gdnq_status st = check_ptrs(sp, N)) return st;
    } else {
      if (gdnq_status st = check_ptrs(sp + 6, N - 6)) return st;
    }
    if (init_codes) {
      const Span ip[] = {{"init_codes", init_codes, bh * L.d_v * L.d_k / (L.q4 ? 2 : 1)},
                         {"init_scales", init_scales, bh * L.d_v * 4}};
      if (gdnq_status st = check_ptrs(ip, 2)) return st;
      if (L.no_requant) {
        for (int i = 0; i < 2; ++i)
          if (overlap(ip[i], sp[6])) return fail(GDNQ_ERR_ALIAS, "%s overlaps state_f32", ip[i].name);
      } else {
        // an in-place continuation (init == final) is allowed; partial overlap is not
        if (init_codes != codes && overlap(ip[0], sp[6])) return fail(GDNQ_ERR_ALIAS, "init_codes partially overlaps codes");
        if (init_scales != scales && overlap(ip[1], sp[7])) return fail(GDNQ_ERR_ALIAS, "init_scales partially overlaps scales");
      }
    }
    for (int i = 5; i < N; ++i)
      for (int j = 0; j < N; ++j)
        if (j != i && overlap(sp[i], sp[j])) return fail(GDNQ_ERR_ALIAS, "%s overlaps %s", sp[i].name, sp[j].name);
    L.beta = beta;
    L.init_codes = init_codes;
    L.init_scales = init_scales;
    L.codes = codes;
    L.scales = scales;
  }
  const size_t need = gdnq::prefill_workspace_bytes(L);
  if (noalloc) {
    if (gdnq_status st = noalloc_workspace(need, workspace, workspace_bytes)) return st;
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDNQ_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace_bytes);
  if (workspace && !aligned16(workspace)) return fail(GDNQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  L.q = q; L.k = k; L.v = v; L.alpha = alpha; L.o = o; L.state_f32 = state_f32; L.workspace = workspace;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_stale_hip_error();
  return launched(L.ssd ? gdnq::launch_prefill_ssd(L, s) : gdnq::launch_prefill_gdn(L, s), "prefill launch", stream);
}

gdnq_status gdnq_prefill_chunked(const gdnq_prefill_params* p, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const int8_t* init_codes, const float* init_scales, void* o,
                                 int8_t* codes, float* scales, float* state_f32,
                                 void* buf_k, void* buf_v, float* buf_alpha, float* buf_beta,
                                 int32_t* fill_out, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_chunked_impl(p, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales, state_f32,
                              buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream, false);
}

gdnq_status gdnq_prefill_chunked_noalloc(const gdnq_prefill_params* p, const void* q, const void* k,
                                         const void* v, const float* alpha, const float* beta,
                                         const int8_t* init_codes, const float* init_scales, void* o,
                                         int8_t* codes, float* scales, float* state_f32,
                                         void* buf_k, void* buf_v, float* buf_alpha, float* buf_beta,
                                         int32_t* fill_out, void* stream) {
  return prefill_chunked_impl(p, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales, state_f32,
                              buf_k, buf_v, buf_alpha, buf_beta, fill_out, nullptr, 0, stream, true);
}

size_t gdnq_prefill_handoff_workspace_size(const gdnq_prefill_params* p) {
  gdnq::PrefillLaunch L;
  if (prefill_validate(p, L, PF_HANDOFF) != GDNQ_OK) return 0;
  return gdnq::prefill_workspace_bytes(L);
}

// Variable lengths: batch = sequences, seqlen = packed tokens in total.
// Positions the chunk kernels see for N new tokens of B sequences (resuming:
// plus up to W - 1 buffered writes each), every window padded to 64
// positions when the window is below 64 or d = 64.
static int64_t mapped_positions(const gdnq::PrefillLaunch& L, int64_t N) {
  const int64_t pre = L.resume ? int64_t(L.B) * (L.W - 1) : 0;
  if (L.W < 64 || L.d_k == 64) return (64 * (N + pre) + L.W - 1) / L.W;
  return N;
}

static gdnq_status varlen_validate(const gdnq_prefill_params* p, gdnq::PrefillLaunch& L) {
  if (gdnq_status st = prefill_validate(p, L, PF_MAPPED)) return st;
  const int64_t pos = mapped_positions(L, L.T);
  if (pos > 0x7fffffffLL) return fail(GDNQ_ERR_SHAPE, "%lld padded positions: at most 2^31 - 1", (long long)pos);
  if ((pos / 64 + L.B) * L.H > 0x7fffffffLL) return fail(GDNQ_ERR_SHAPE, "too many chunks");
  L.varlen = true;
  return GDNQ_OK;
}

size_t gdnq_prefill_varlen_workspace_size(const gdnq_prefill_params* p) {
  gdnq::PrefillLaunch L;
  if (varlen_validate(p, L) != GDNQ_OK) return 0;
  return gdnq::prefill_workspace_bytes(L);
}

static gdnq_status prefill_handoff_impl(gdnq::PrefillLaunch& L, const int32_t* cu_seqlens,
                                        const int32_t* fill_in, const void* q, const void* k, const void* v, const float* alpha,
                                        const float* beta, const int8_t* init_codes, const float* init_scales,
                                        void* o, int8_t* codes, float* scales, void* buf_k, void* buf_v,
                                        float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                        void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  if (L.B == 0) return ok();
  // token-indexed arrays: B x T tokens, or T packed tokens of variable-length sequences
  const size_t bth = (cu_seqlens ? size_t(1) : size_t(L.B)) * L.T * L.H, bh = size_t(L.B) * L.H;
  const size_t eo = L.out_bf16 ? 2 : 4, W = size_t(L.W);
  // window buffer bytes per key / value vector: fp32, bf16, or E4M3 codes
  // (the per-vector fp32 scales follow all the codes in the same allocation)
  const size_t bk_bytes = L.buf_fp8 ? bh * W * (L.d_k + 4) : bh * W * L.d_k * (L.buf_bf16 ? 2 : 4);
  const size_t bv_bytes = L.buf_fp8 ? bh * W * (L.d_v + 4) : bh * W * L.d_v * (L.buf_bf16 ? 2 : 4);
  if ((init_codes == nullptr) != (init_scales == nullptr))
    return fail(GDNQ_ERR_NULL, "init_codes and init_scales must be both NULL or both set");
  const Span sp[] = {{"q", q, bth * L.d_k * 2},          {"k", k, bth * L.d_k * 2},
                     {"v", v, bth * L.d_v * 2},          {"alpha", alpha, bth * 4},
                     {"beta", beta, bth * 4},            {"o", o, bth * L.d_v * eo},
                     {"codes", codes, bh * L.d_v * L.d_k / (L.q4 ? 2 : 1)}, {"scales", scales, bh * L.d_v * 4},
                     {"buf_k", buf_k, bk_bytes},         {"buf_v", buf_v, bv_bytes},
                     {"buf_alpha", buf_alpha, bh * W * 4}, {"buf_beta", buf_beta, bh * W * 4},
                     {"fill_out", fill_out, size_t(L.B) * 4}};
  constexpr int N = sizeof(sp) / sizeof(sp[0]);
  if (L.T > 0) {
    if (gdnq_status st = check_ptrs(sp, N)) return st;
  } else {
    if (gdnq_status st = check_ptrs(sp + 6, N - 6)) return st;
  }
  if (init_codes) {
    const Span ip[] = {{"init_codes", init_codes, bh * L.d_v * L.d_k / (L.q4 ? 2 : 1)},
                       {"init_scales", init_scales, bh * L.d_v * 4}};
    if (gdnq_status st = check_ptrs(ip, 2)) return st;
    if (init_codes != codes && overlap(ip[0], sp[6])) return fail(GDNQ_ERR_ALIAS, "init_codes partially overlaps codes");
    if (init_scales != scales && overlap(ip[1], sp[7])) return fail(GDNQ_ERR_ALIAS, "init_scales partially overlaps scales");
  }
  for (int i = 5; i < N; ++i)  // every written buffer is disjoint from every other
    for (int j = 0; j < N; ++j)
      if (j != i && overlap(sp[i], sp[j])) return fail(GDNQ_ERR_ALIAS, "%s overlaps %s", sp[i].name, sp[j].name);
  if (cu_seqlens) {
    if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return fail(GDNQ_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
    const Span cs{"cu_seqlens", cu_seqlens, (size_t(L.B) + 1) * 4};
    for (int i = 5; i < N; ++i)
      if (overlap(cs, sp[i])) return fail(GDNQ_ERR_ALIAS, "cu_seqlens overlaps %s", sp[i].name);
  }
  if (L.resume) {  // fill_in is read before anything is written: it may be fill_out itself
    if (!fill_in) return fail(GDNQ_ERR_NULL, "fill_in is NULL");
    if (reinterpret_cast<uintptr_t>(fill_in) & 3u) return fail(GDNQ_ERR_ALIGN, "fill_in is not 4-byte aligned");
    const Span fs{"fill_in", fill_in, size_t(L.B) * 4};
    for (int i = 5; i < N; ++i)
      if (!(i == N - 1 && fill_in == fill_out) && overlap(fs, sp[i]))
        return fail(GDNQ_ERR_ALIAS, "fill_in overlaps %s", sp[i].name);
  }
  const size_t need = gdnq::prefill_workspace_bytes(L);
  if (noalloc) {
    if (gdnq_status st = noalloc_workspace(need, workspace, workspace_bytes)) return st;
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDNQ_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace_bytes);
  if (workspace && !aligned16(workspace)) return fail(GDNQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  L.cu_seqlens = cu_seqlens;
  L.fill_in = fill_in;
  L.q = q; L.k = k; L.v = v; L.alpha = alpha; L.beta = beta; L.o = o;
  L.init_codes = init_codes; L.init_scales = init_scales; L.codes = codes; L.scales = scales;
  L.workspace = workspace;
  L.buf_k = buf_k; L.buf_v = buf_v; L.buf_alpha = buf_alpha; L.buf_beta = buf_beta; L.fill_out = fill_out;
  clear_stale_hip_error();
  return launched(gdnq::launch_prefill_gdn(L, static_cast<hipStream_t>(stream)), "prefill hand-over launch", stream);
}

gdnq_status gdnq_prefill_handoff(const gdnq_prefill_params* p, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const int8_t* init_codes, const float* init_scales, void* o,
                                 int8_t* codes, float* scales, void* buf_k, void* buf_v,
                                 float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  gdnq::PrefillLaunch L;
  if (gdnq_status st = prefill_validate(p, L, PF_HANDOFF)) return st;
  return prefill_handoff_impl(L, nullptr, nullptr, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales,
                              buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream);
}

gdnq_status gdnq_prefill_varlen(const gdnq_prefill_params* p, const int32_t* cu_seqlens, const void* q,
                                const void* k, const void* v, const float* alpha, const float* beta,
                                const int8_t* init_codes, const float* init_scales, void* o,
                                int8_t* codes, float* scales, void* buf_k, void* buf_v,
                                float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  gdnq::PrefillLaunch L;
  if (gdnq_status st = varlen_validate(p, L)) return st;
  if (L.B > 0 && !cu_seqlens) return fail(GDNQ_ERR_NULL, "cu_seqlens is NULL");
  return prefill_handoff_impl(L, cu_seqlens, nullptr, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales,
                              buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream);
}

// Resuming from decode: batch = sequences; seqlen = new tokens per sequence,
// or packed new tokens in total with cu_seqlens.
static gdnq_status resume_validate(const gdnq_prefill_params* p, bool varlen, gdnq::PrefillLaunch& L) {
  if (gdnq_status st = prefill_validate(p, L, PF_MAPPED)) return st;
  const int64_t tokens = varlen ? int64_t(L.T) : int64_t(L.B) * L.T;
  if (tokens > 0x7fffffffLL) return fail(GDNQ_ERR_SHAPE, "%lld new tokens: at most 2^31 - 1", (long long)tokens);
  L.varlen = varlen;
  L.resume = true;
  const int64_t pos = mapped_positions(L, tokens);
  if (pos > 0x7fffffffLL) return fail(GDNQ_ERR_SHAPE, "%lld padded positions: at most 2^31 - 1", (long long)pos);
  if ((pos / 64 + 2 * int64_t(L.B)) * L.H > 0x7fffffffLL) return fail(GDNQ_ERR_SHAPE, "too many chunks");
  return GDNQ_OK;
}

size_t gdnq_prefill_resume_workspace_size(const gdnq_prefill_params* p, int32_t varlen) {
  gdnq::PrefillLaunch L;
  if (resume_validate(p, varlen != 0, L) != GDNQ_OK) return 0;
  return gdnq::prefill_workspace_bytes(L);
}

gdnq_status gdnq_prefill_resume(const gdnq_prefill_params* p, const int32_t* cu_seqlens, const int32_t* fill_in,
                                const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, void* o, int8_t* codes, float* scales, void* buf_k,
                                void* buf_v, float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  gdnq::PrefillLaunch L;
  if (gdnq_status st = resume_validate(p, cu_seqlens != nullptr, L)) return st;
  if (!codes || !scales) return fail(GDNQ_ERR_NULL, "codes and scales (the stored state) are required");
  return prefill_handoff_impl(L, cu_seqlens, fill_in, q, k, v, alpha, beta, codes, scales, o, codes, scales,
                              buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream);
}

}  // extern "C"
