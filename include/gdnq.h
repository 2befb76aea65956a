/*
 * gdnq.h -- C ABI of the int8-state gated delta-rule (Gated DeltaNet) library
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes
 *   The recurrence (the pages name it; this is the standard gated delta rule)
 *       S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *       o_t = S_t q_t,                      S in R^{d_v x d_k},
 *   with the state held as int8 codes plus one fp32 scale per row (a row is
 *   one v index: d_k codes).  The state is requantized once per window of W
 *   tokens; inside a window the window's writes (k, v, alpha, beta) are kept
 *   in fp32 and replayed on top of the dequantized state.
 *     - "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
 *       Quantization", abstract: 8-bit recurrent state, per-window
 *       quantization (quantize once at the window's end; outputs inside the
 *       window from the fixed low-bit state plus high-precision buffered
 *       updates).
 *     - "Low-Bit GDN Recurrent-State Quantization: Global Gradient-aware
 *       Allocation and Pure-Write Sliding Windows", abstract: buffered writes
 *       go through the full GDN transition and are merged into the low-bit
 *       state when they leave the window.
 *     - "LinQuant: Functional Invariances for Low-Precision Linear
 *       Recurrences", abstract: chunkwise-parallel prefill as dense matrix
 *       products; rotations as invariances; SSD (Mamba-2) prefill with
 *       low-precision operands.
 *     - "Influence-Inspired Spectral Rotations for Extreme Low-Bit LLM
 *       Quantization", abstract: the Walsh-Hadamard rotation.
 *
 * Codec (all entry points): per row, scale = max|x| / 127 (fp32, IEEE
 * division); code = clamp(round_half_even(x / scale), -127, 127); a row with
 * max|x| = 0 gets scale 0 and codes 0.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers, owned by the caller.  The library
 *     allocates no device memory and keeps no per-call state.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL means the default stream).
 *   - Arguments are validated on the host before anything is launched.  On any
 *     status other than GDNQ_OK nothing has been launched and nothing written;
 *     gdnq_last_error() gives a one-line reason (thread-local).
 *   - Every pointer must be 16-byte aligned; layouts are dense row-major with
 *     the innermost dimension listed last.
 *   - Floating-point data errors (NaN/Inf inputs, ||k|| != 1, beta outside
 *     [0,1]) are not checked; results are then unspecified.
 *   - No C++ exception crosses this interface.  Calls are reentrant.
 *   - Device faults surface on the caller's next synchronisation, unless
 *     the environment variable GDNQ_SYNC_DEBUG is "1" when the library is
 *     loaded: then every call waits for its own kernels on its stream before
 *     it returns, and reports a fault of theirs as GDNQ_ERR_HIP with the
 *     call's name in gdnq_last_error() (a debugging aid: it serializes the
 *     caller's stream).  gdnq_sync_debug() tells which mode is in force.
 */
#ifndef GDNQ_H
#define GDNQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDNQ_OK = 0,
  GDNQ_ERR_NULL = 1,      /* a required pointer is NULL                        */
  GDNQ_ERR_SHAPE = 2,     /* unsupported size / size combination              */
  GDNQ_ERR_DTYPE = 3,     /* unsupported dtype code                            */
  GDNQ_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                  */
  GDNQ_ERR_ALIAS = 5,     /* an output aliases an input it must not alias      */
  GDNQ_ERR_WORKSPACE = 6, /* workspace missing or too small                    */
  GDNQ_ERR_HIP = 7,       /* the HIP runtime refused the launch               */
  GDNQ_ERR_FLAGS = 8      /* unknown or unsupported flag bits                  */
} gdnq_status;

/* Largest prefill window (tokens). */
#define GDNQ_MAX_WINDOW (1 << 24)

/* Element types of q, k, v (in_dtype) and of o (out_dtype). */
enum { GDNQ_F32 = 0, GDNQ_BF16 = 1 };

/* Flag bits. */
enum {
  GDNQ_FLAG_WHT = 1u,     /* rotate q and k by the normalised Walsh-Hadamard
                             matrix H/sqrt(d_k) (Sylvester order) before use;
                             the state then lives in the rotated basis S H    */
  GDNQ_FLAG_SSD = 2u,     /* prefill only: scalar-decay SSD recurrence
                             S_t = a_t S_{t-1} + v_t k_t^T (no delta term);
                             state kept in fp32, not quantized                */
  GDNQ_FLAG_INT8_QK = 4u, /* prefill + SSD only: quantize each token's
                             (rotated) q and k row to int8 with the codec
                             above and use the dequantized operands         */
  GDNQ_FLAG_NO_REQUANT = 8u, /* gdnq_prefill_chunked, GDN only (a reference
                             mode for tests): never requantize; the state
                             starts from init_codes/init_scales (or zero) and
                             the final fp32 state goes to state_f32 (codes
                             and scales NULL); any T (window ignored)        */
  GDNQ_FLAG_BUF_BF16 = 16u, /* decode and the prefill hand-over, varlen and
                             resume calls: the window buffer keeps keys and
                             values as bf16 (buf_k, buf_v element type).  A
                             token's write enters its own step exactly and is
                             stored rounded to nearest even, so later steps
                             and the window's close replay the rounded write;
                             alpha and beta stay fp32.  Lossless when q, k, v
                             are bf16 and GDNQ_FLAG_WHT is off.              */
  GDNQ_FLAG_BUF_FP8 = 32u, /* decode and the prefill hand-over, varlen and
                             resume calls: the window buffer keeps keys and
                             values as FP8 vector pairs (Low-Bit GDN ...,
                             abstract): each buffered key and each value is
                             OCP E4M3 codes (bias 7, largest finite 448) with
                             one fp32 scale absmax/448; a code is the E4M3
                             value nearest to x/scale (IEEE fp32 division,
                             ties to even).  The token's own write enters its
                             step exactly and is stored quantized.  Layout:
                             buf_k = B*H*W*d_k code bytes, then B*H*W fp32
                             scales; buf_v likewise with d_v.  Exclusive with
                             GDNQ_FLAG_BUF_BF16.                            */
  GDNQ_FLAG_SLIDING = 128u, /* decode only: the Pure-Write sliding window
                             (Low-Bit GDN ..., abstract) instead of the
                             tumbling one.  The buffer is a ring of the last W
                             raw writes per head; codes/scales hold the
                             historical state H.  Per token: H' = deq(H) A_t,
                             plus beta_l v_l k~_l^T for the write l that leaves
                             a full window (k~_l: its key through every later
                             transition, A_j = alpha_j (I - beta_j k_j
                             k_j^T)); o = (H' + window) q; H = quantize(H')
                             at every token (codes and scales of every
                             sequence are rewritten); the token's write takes
                             the ring slot of the write that left.  fill is
                             in [0, 2W): below W the window holds `fill`
                             writes in slots 0..fill-1; from W on it is full
                             and its oldest write is in slot fill - W.
                             fill_out = fill + 1 below W, else W + (fill - W
                             + 1) mod W.  fp32 window buffer and 8-bit state
                             only (exclusive with GDNQ_FLAG_BUF_BF16,
                             GDNQ_FLAG_BUF_FP8, GDNQ_FLAG_STATE_4BIT).      */
  GDNQ_FLAG_STATE_4BIT = 64u /* quantize, decode and GDN prefill (all its
                             entry points): the uniform 4-bit state
                             (Low-Bit GDN ..., abstract: the "@4" budget of
                             four bits per state entry).  The codec above with
                             127 replaced by 7: scale = max|x| / 7, codes =
                             clamp(round_half_even(x / scale), -7, 7).  Codes
                             are packed two per byte: row-major [rows, d_k/2]
                             bytes, column 2j in the low nibble of byte j,
                             column 2j+1 in the high nibble, each a two's
                             complement nibble.  Scales are unchanged.      */
};

/* ------------------------------------------------------------------------
 * gdnq_quantize_state -- codec (int8 codes + per-row fp32 scales).
 *   LeapQuant, abstract (8-bit recurrent state).
 *
 *   S       [rows, d_k] fp32, read only
 *   codes   [rows, d_k] int8, written ([rows, d_k/2] bytes of packed 4-bit
 *           codes under GDNQ_FLAG_STATE_4BIT)
 *   scales  [rows]      fp32, written
 *   flags   GDNQ_FLAG_WHT (rotate each row x -> H x / sqrt(d_k) first,
 *           i.e. quantize S H, the state in the rotated basis) and/or
 *           GDNQ_FLAG_STATE_4BIT
 *   d_k in {64, 128}; rows >= 0 (rows == 0 is a no-op).
 *   Errors: NULL (any pointer, rows > 0), SHAPE, ALIGN, FLAGS, HIP.
 * ------------------------------------------------------------------------ */
gdnq_status gdnq_quantize_state(const float* S, int64_t rows, int32_t d_k, int8_t* codes,
                                float* scales, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_decode_step -- one token per sequence, per-window quantized state.
 *   LeapQuant, abstract (per-window quantization; outputs from the low-bit
 *   state plus buffered high-precision updates); Low-Bit GDN ..., abstract
 *   (writes propagate through the full transition, merge on window exit).
 *
 *   For every sequence b with f = fill_in[b] writes already buffered (the
 *   same f for all its heads), and every head h:
 *     S := dequant(codes, scales); replay buffered writes 0..f-1 on S (oldest
 *     first); apply the current token; o = S q.
 *     If f + 1 < W: append (k, v, alpha, beta) of the token to slot f of the
 *       buffer (k in the rotated basis under GDNQ_FLAG_WHT), fill_out[b] = f+1;
 *       codes and scales are left untouched.
 *     If f + 1 == W (window closes): codes and scales of the sequence are
 *       rewritten with the requantized S; fill_out[b] = 0.  Buffer contents
 *       at slots >= fill_out are unspecified afterwards.
 *   The output of a closing token uses S before requantization.
 *
 *   0 <= p->batch B <= 1024 (0: no-op), p->heads H >= 1, p->d_k, p->d_v in {64,128},
 *   1 <= p->window W <= 64, p->in_dtype (q,k,v) and p->out_dtype (o) in
 *   {GDNQ_F32, GDNQ_BF16}, p->flags a combination of GDNQ_FLAG_WHT, at
 *   most one of GDNQ_FLAG_BUF_BF16, GDNQ_FLAG_BUF_FP8 (the low-precision
 *   window buffers; the Low-Bit GDN page keeps recent writes in FP8), and
 *   GDNQ_FLAG_STATE_4BIT (the state as packed 4-bit codes, requantized
 *   with the 4-bit codec when a window closes), or GDNQ_FLAG_SLIDING (the
 *   Pure-Write sliding window; see the flag: fill_in in [0, 2W) then).
 *     q, k      [B,H,d_k] in_dtype      v [B,H,d_v] in_dtype
 *     alpha, beta [B,H] fp32
 *     codes     [B,H,d_v,d_k] int8      scales [B,H,d_v] fp32   (in/out)
 *               ([B,H,d_v,d_k/2] bytes under GDNQ_FLAG_STATE_4BIT)
 *     buf_k     [B,H,W,d_k]             buf_v [B,H,W,d_v]       (in/out)
 *               fp32, or bf16 under GDNQ_FLAG_BUF_BF16, or under
 *               GDNQ_FLAG_BUF_FP8 E4M3 bytes [B,H,W,d] followed by fp32
 *               scales [B,H,W] in the same buffer
 *     buf_alpha, buf_beta [B,H,W] fp32                           (in/out)
 *     fill_in   [B] int32 in [0, W-1]   fill_out [B] int32 (written)
 *     o         [B,H,d_v] out_dtype (written)
 *   fill_in and fill_out must be distinct buffers (every head of a sequence
 *   reads fill_in while the call runs): equal pointers give GDNQ_ERR_ALIAS.
 *   A fill_in value outside [0, W-1] is a data error (result unspecified,
 *   memory accesses stay inside the buffers).
 *   Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, FLAGS, HIP.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch, heads, d_k, d_v, window;
  int32_t in_dtype, out_dtype;
  uint32_t flags;
} gdnq_decode_params;

gdnq_status gdnq_decode_step(const gdnq_decode_params* p, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta,
                             int8_t* codes, float* scales, void* buf_k, void* buf_v,
                             float* buf_alpha, float* buf_beta, const int32_t* fill_in,
                             int32_t* fill_out, void* o, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_prefill_chunked -- chunkwise-parallel prefill.
 *   LinQuant, abstract (chunkwise-parallel prefill as dense matrix products;
 *   SSD prefill with int8 operands; rotations); LeapQuant, abstract
 *   (requantize once per window).
 *
 *   GDN (flags without GDNQ_FLAG_SSD): the gated delta rule over T tokens
 *   from the stored state (init_codes/init_scales, or zero when both are
 *   NULL), requantizing at every window end, windows aligned to token 0.
 *   Supported: d_k = d_v in {128, 64} (GDNQ_FLAG_WHT at 128 only), chunk
 *   in {16, 32, 64}, any window 1 <= W <= GDNQ_MAX_WINDOW, T a multiple of
 *   W when the window-buffer arguments are NULL.  The kernels run every window as
 *   whole 64-position chunks (a window that is not a multiple of 64 is
 *   padded at its end with writes that leave the state unchanged; d = 64
 *   runs as a zero-padded d = 128 head; between the chunks of one window
 *   the state stays fp32), so the result depends on the window, not on the
 *   chunk, which is a blocking hint.  Padded runs need a larger workspace.
 *   Writes o and the final codes/scales (the state after the last window);
 *   state_f32 must be NULL, except under GDNQ_FLAG_NO_REQUANT, which
 *   writes the final fp32 state there instead of codes/scales (which must
 *   then be NULL; any T; init_codes must not overlap state_f32; the state
 *   is in the rotated basis under GDNQ_FLAG_WHT).
 *   Flags: GDNQ_FLAG_STATE_4BIT (init_codes and
 *   codes then hold packed 4-bit codes, [B,H,d_v,d_k/2] bytes, and every
 *   window end requantizes with the 4-bit codec) and/or GDNQ_FLAG_WHT: every
 *   q and k row is rotated by H/sqrt(128) in fp32 and rounded to bf16
 *   (nearest even), the operand precision of the chunk products; the state
 *   (init_codes in, codes out) lives in the rotated basis S H.
 *
 *   SSD (GDNQ_FLAG_SSD): S_t = a_t S_{t-1} + v_t k_t^T from a zero state, no
 *   requantization (window ignored); beta, init_codes, init_scales, codes and
 *   scales must be NULL; writes o and the final fp32 state (in the rotated
 *   basis under GDNQ_FLAG_WHT).  Supported: d_k, d_v in {64, 128},
 *   chunk = 64, T a multiple of 64.  Flags: GDNQ_FLAG_INT8_QK and/or
 *   GDNQ_FLAG_WHT (each q and k row rotated by H/sqrt(d_k) in fp32, then
 *   quantized to int8 with INT8_QK, else rounded to bf16 (nearest even), the
 *   operand precision of the products; workspace: the rotated rows).  At
 *   d_k = 64 the q and k rows are widened to 128 with zeros (after the
 *   rotation and quantization, so neither sees the zeros) and the state is
 *   built 128 wide and its first 64 columns copied to state_f32; the
 *   workspace then holds the widened rows (bf16 unless INT8_QK, also with
 *   neither flag) and, from the next 256-byte boundary, B*H*d_v*128 fp32.
 *
 *   p->in_dtype must be GDNQ_BF16, p->out_dtype GDNQ_BF16 or GDNQ_F32.
 *     q, k   [B,T,H,d_k] in_dtype     v [B,T,H,d_v] in_dtype
 *     alpha  [B,T,H] fp32             beta [B,T,H] fp32 (GDN only)
 *     init_codes [B,H,d_v,d_k] int8, init_scales [B,H,d_v] fp32 (GDN; may
 *       alias codes/scales for an in-place continuation)
 *     o      [B,T,H,d_v] out_dtype    (written)
 *     codes  [B,H,d_v,d_k] int8, scales [B,H,d_v] fp32 (GDN, written)
 *     state_f32 [B,H,d_v,d_k] fp32 (SSD and GDNQ_FLAG_NO_REQUANT, written)
 *     buf_k, buf_v, buf_alpha, buf_beta, fill_out: decode's window buffer
 *       and fills.  All NULL: whole windows only (T a multiple of W; SSD
 *       and GDNQ_FLAG_NO_REQUANT have no windows).  Any of them set, or a
 *       windowed GDN call with T not a multiple of W: all five required and
 *       the call is gdnq_prefill_handoff below (GDN, decode's window W in
 *       1..64, state_f32 NULL, no GDNQ_FLAG_NO_REQUANT; the buffer format
 *       flags GDNQ_FLAG_BUF_BF16 / GDNQ_FLAG_BUF_FP8 apply): codes/scales
 *       take the state at the last window boundary, the T mod W writes of
 *       the open window go to slots 0.. of the buffer and fill_out to
 *       T mod W, so that gdnq_decode_step continues the sequence.
 *   workspace: gdnq_prefill_workspace_size(p) bytes of device memory (may be
 *   NULL when that size is 0).
 *   Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, FLAGS, WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch, seqlen, heads, d_k, d_v, chunk, window;
  int32_t in_dtype, out_dtype;
  uint32_t flags;
} gdnq_prefill_params;

/* Workspace bytes of gdnq_prefill_chunked for these parameters (0 when
 * they are invalid): with T a multiple of W, enough both without and with
 * the window-buffer arguments. */
size_t gdnq_prefill_workspace_size(const gdnq_prefill_params* p);

gdnq_status gdnq_prefill_chunked(const gdnq_prefill_params* p, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const int8_t* init_codes, const float* init_scales, void* o,
                                 int8_t* codes, float* scales, float* state_f32,
                                 void* buf_k, void* buf_v, float* buf_alpha, float* buf_beta,
                                 int32_t* fill_out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_prefill_chunked_noalloc -- gdnq_prefill_chunked for callers that
 *   cannot allocate device memory: code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc.  Same parameters,
 *   results, layouts and errors as gdnq_prefill_chunked, without the
 *   workspace arguments: the workspace is a fixed array of
 *   GDNQ_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 *   every GPU it runs on, from load until the process ends.  The call uses
 *   the array of the current device (the stream must belong to it) and
 *   allocates nothing, neither device nor host memory.
 *     - A call that needs more workspace than GDNQ_NOALLOC_SCRATCH_BYTES
 *       (gdnq_prefill_workspace_size(p) bounds it) is rejected with
 *       GDNQ_ERR_WORKSPACE before anything is launched (e.g. GDN: 15,616 bytes per chunk-head,
 *       so B * (T / 64) * H <= 4297; SSD with GDNQ_FLAG_INT8_QK: 264 bytes
 *       per token-head).
 *     - Every call on one GPU shares that GPU's array: calls that overlap
 *       in time on one GPU (on different streams, or from different host
 *       threads without ordering) race and give unspecified results.
 *       Calls ordered on one stream are safe.  Nothing in the array needs
 *       to start at zero; it keeps the last call's contents.
 *   Errors: as gdnq_prefill_chunked (WORKSPACE: too large for the array;
 *   HIP: the array's device address could not be queried).
 * ------------------------------------------------------------------------ */
#define GDNQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gdnq_status gdnq_prefill_chunked_noalloc(const gdnq_prefill_params* p, const void* q, const void* k,
                                         const void* v, const float* alpha, const float* beta,
                                         const int8_t* init_codes, const float* init_scales, void* o,
                                         int8_t* codes, float* scales, float* state_f32,
                                         void* buf_k, void* buf_v, float* buf_alpha, float* buf_beta,
                                         int32_t* fill_out, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_prefill_handoff -- GDN prefill of T tokens (any T >= 0) that leaves
 *   its last, open window in decode's window buffer, so that
 *   gdnq_decode_step continues the sequence.  LeapQuant, abstract (outputs
 *   inside a window from the fixed low-bit state plus buffered writes;
 *   requantize once at the window's end).
 *
 *   Same recurrence, parameters and layouts as gdnq_prefill_chunked in GDN
 *   mode (flags GDNQ_FLAG_STATE_4BIT and/or GDNQ_FLAG_WHT, d_k = d_v in
 *   {128, 64} (the rotation at 128 only), chunk in {16, 32, 64}, in_dtype
 *   bf16), with decode's window W in 1 .. 64, except that p->seqlen T need
 *   not be a multiple of W.  With r = T mod W:
 *     o          [B,T,H,d_v] out_dtype, every token (written)
 *     codes, scales: the state at the last window boundary (token T - r)
 *     buf_k, buf_v  decode's window buffer [B,H,W,d] in the format the
 *                flags select (slots < r written): fp32 (no flag), bf16
 *                (GDNQ_FLAG_BUF_BF16: the bf16 inputs themselves), or FP8
 *                vector pairs (GDNQ_FLAG_BUF_FP8: E4M3 codes, then the
 *                per-vector fp32 scales, encoded as decode's append does);
 *                under GDNQ_FLAG_WHT the keys are the rotated ones the
 *                prefill used (rounded to bf16), and the state is in the
 *                rotated basis, as decode with GDNQ_FLAG_WHT keeps them
 *     buf_alpha, buf_beta [B,H,W] fp32                        (slots < r written)
 *     fill_out   [B] int32 = r for every sequence (written)
 *   i.e. exactly decode's state after its last r steps: a decode step with
 *   fill_in = fill_out and the same buffer and rotation flags continues the
 *   sequence.
 *   workspace: gdnq_prefill_handoff_workspace_size(p) bytes.
 *   Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, FLAGS, WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
size_t gdnq_prefill_handoff_workspace_size(const gdnq_prefill_params* p);

gdnq_status gdnq_prefill_handoff(const gdnq_prefill_params* p, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const int8_t* init_codes, const float* init_scales, void* o,
                                 int8_t* codes, float* scales, void* buf_k, void* buf_v,
                                 float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_prefill_varlen -- gdnq_prefill_handoff over a packed batch of
 *   sequences of different lengths (LeapQuant, abstract: the same
 *   recurrence, window buffer and boundary requantization per sequence).
 *
 *   p->batch B = number of sequences, p->seqlen T = total packed tokens;
 *   the other fields as for gdnq_prefill_handoff (decode's window W in
 *   1 .. 64, d in {64, 128}, optional rotation).  Below W = 64 or at d = 64
 *   every sequence is padded on the device (its whole windows to 64
 *   positions, its open window unpadded).
 *     cu_seqlens [B+1] int32, device: sequence b holds packed tokens
 *                cu_seqlens[b] .. cu_seqlens[b+1]-1.  Expected
 *                0 = cu[0] <= cu[1] <= ... <= cu[B] = T.  The kernels take
 *                the running maximum of the values clamped to [0, T], so
 *                malformed offsets never reach outside the buffers; what
 *                they compute for such input is not specified.
 *     q, k [T,H,128] bf16   v [T,H,128] bf16   alpha, beta [T,H] fp32
 *     o    [T,H,128] out_dtype (every token of every sequence written)
 *     init_codes, init_scales, codes, scales, buf_*: per sequence, as in
 *                gdnq_prefill_handoff ([B,H,...]).
 *     fill_out   [B] int32 = len_b mod 64 per sequence (written)
 *   A sequence of length 0 copies its initial state (or zeros) to codes,
 *   scales and sets its fill to 0.
 *   workspace: gdnq_prefill_varlen_workspace_size(p) bytes (bounded by
 *   floor(T/64) + B chunks per head, plus 4 (4B+2) bytes of sequence map).
 *   Errors: NULL, SHAPE, DTYPE, ALIGN (cu_seqlens: 4 bytes), ALIAS, FLAGS,
 *   WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
size_t gdnq_prefill_varlen_workspace_size(const gdnq_prefill_params* p);

gdnq_status gdnq_prefill_varlen(const gdnq_prefill_params* p, const int32_t* cu_seqlens, const void* q,
                                const void* k, const void* v, const float* alpha, const float* beta,
                                const int8_t* init_codes, const float* init_scales, void* o,
                                int8_t* codes, float* scales, void* buf_k, void* buf_v,
                                float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_prefill_resume -- GDN prefill that continues sequences from their
 *   decode state at any fill: windows need not start at a chunk boundary
 *   (LeapQuant, abstract: outputs inside a window from the fixed low-bit
 *   state plus the buffered writes; one requantization when the window is
 *   full).  For each sequence the open window's fill_in[b] buffered writes
 *   and its new tokens form one sequence whose windows of W positions start
 *   at the first buffered write, so the first window closes after
 *   W - fill_in[b] new tokens, exactly as decode would close it.
 *
 *   p->batch B = sequences; p->seqlen = new tokens per sequence (cu_seqlens
 *   NULL, q [B,T,H,d] ...) or packed new tokens in total (cu_seqlens as for
 *   gdnq_prefill_varlen, q [T,H,d] ...).  GDN mode only (flags
 *   GDNQ_FLAG_STATE_4BIT and/or GDNQ_FLAG_WHT, with one window-buffer format
 *   flag as for gdnq_prefill_handoff; d_k = d_v = d in {64, 128}, the
 *   rotation at 128 only; p->window = decode's window W in 1 .. 64; chunk a
 *   blocking hint in {16, 32, 64}; in_dtype bf16).  Below W = 64 or at
 *   d = 64 every sequence is padded on the device (whole windows to 64
 *   positions, the open window unpadded).
 *     fill_in    [B] int32, device: buffered writes per sequence (0..W-1;
 *                other values are clamped into that range).  It may be the
 *                same array as fill_out.
 *     codes, scales [B,H,d,d] int8 / [B,H,d] fp32: the state at the
 *                last window boundary on entry, at the new last boundary on
 *                return (updated in place).
 *     buf_k, buf_v [B,H,W,d] (fp32, bf16 or FP8 vector pairs, as the
 *                flags select), buf_alpha, buf_beta [B,H,W] fp32:
 *                decode's window buffer on entry (slots < fill_in read; the
 *                stored keys and values -- code * scale for FP8 -- enter the
 *                chunk products rounded to bf16, exact when decode's inputs
 *                were bf16 and the buffer fp32 or bf16), the new open
 *                window's writes on return (slots < fill_out).
 *     o          new tokens' outputs, out_dtype (every new token written;
 *                the buffered writes have none: decode gave them).
 *     fill_out   [B] int32 = (fill_in + new tokens) mod W (written).
 *   workspace: gdnq_prefill_resume_workspace_size(p, cu_seqlens != NULL).
 *   Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, FLAGS, WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
size_t gdnq_prefill_resume_workspace_size(const gdnq_prefill_params* p, int32_t varlen);

gdnq_status gdnq_prefill_resume(const gdnq_prefill_params* p, const int32_t* cu_seqlens, const int32_t* fill_in,
                                const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, void* o, int8_t* codes, float* scales, void* buf_k,
                                void* buf_v, float* buf_alpha, float* buf_beta, int32_t* fill_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gdnq_decode_set_schedule -- tuning hook of gdnq_decode_step's persistent
 *   launch (not part of the method; results do not depend on it).
 *   grid: workgroups of the persistent grid; open_waves: waves that take the
 *   sequences whose window stays open.  0 restores the default of either.
 *   The initial values come from the environment variables GDNQ_DECODE_GRID
 *   and GDNQ_DECODE_OPEN_WAVES, read once when the library is loaded.  The
 *   setting is process-wide and applies to launches made after the call.
 *   Errors: SHAPE (a negative value).
 * ------------------------------------------------------------------------ */
gdnq_status gdnq_decode_set_schedule(int32_t grid, int32_t open_waves);

/* Status text, last error detail (thread-local, "" if none), library version,
 * and 1 when GDNQ_SYNC_DEBUG=1 was set at load (every call synchronizes its
 * stream and reports its kernels' faults itself), else 0. */
const char* gdnq_status_string(gdnq_status s);
const char* gdnq_last_error(void);
int32_t gdnq_version(void);
int32_t gdnq_sync_debug(void);

#ifdef __cplusplus
}
#endif
#endif /* GDNQ_H */
