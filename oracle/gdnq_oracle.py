"""Plain CPU oracle for the int8-state gated delta-rule (GDN) recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports, links or calls
this module; only tests, the smoke check and the benchmark's CPU-baseline leg
do.  It is written for readability, not speed: numpy, explicit loops over
tokens, one library primitive (matmul / solve) per algebraic step.

Sources (cited by page title and section; the pages give no formulas):
  [LQ]  "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
        Quantization", abstract: 8-bit recurrent state; per-window
        quantization that leaps over a window of tokens and quantizes the
        state once at the window's end, computing outputs inside the window
        from the fixed low-bit state plus high-precision buffered updates;
        the recurrence family is Gated DeltaNet.
  [PW]  "Low-Bit GDN Recurrent-State Quantization: Global Gradient-aware
        Allocation and Pure-Write Sliding Windows", abstract: recent writes
        are kept apart, propagated through the full GDN state transition and
        merged into the low-bit historical state only when they leave the
        window.
  [LIN] "LinQuant: Functional Invariances for Low-Precision Linear
        Recurrences", abstract: chunkwise-parallel prefill casts the
        recurrence as dense matrix multiplications; rotations are among the
        invariances that keep the full-precision result; SSD (Mamba-2)
        prefill with low-precision operands.
  [BBT] "Influence-Inspired Spectral Rotations for Extreme Low-Bit LLM
        Quantization", abstract: the Walsh-Hadamard rotation as a
        math-invariant transformation applied before quantization.

The recurrence (the pages name it only; this is the standard gated delta
rule with scalar decay alpha and write strength beta):
    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,            S in R^{d_v x d_k}.
Scalar-decay SSD variant ([LIN], Mamba-2):  S_t = a_t S_{t-1} + v_t k_t^T.

Readings taken where the pages are silent (each is also listed in the
design notes):
  * codec: per row (one row = one v index, d_k entries) symmetric absmax/127,
    round-half-to-even, fp32 scale; an all-zero row gets scale 0 and codes 0;
    codes clamp to [-127, 127].  The decision x/scale is taken in fp32 with
    an IEEE-rounded division.
  * windows are tumbling and aligned to token 0; the output of the token that
    closes a window comes from the fp32 state before requantization; the
    buffered writes are replayed on top of the dequantized state (the
    low-bit state takes the window's transitions, [PW]).
  * q and k are used as given (no 1/sqrt(d) scaling, no normalisation).
  * the uniform 4-bit state (qmax = 7): the same codec with 15 levels
    (scale = absmax/7, codes in [-7, 7]); windows and replay unchanged.
  * continuing a sequence by prefill when f writes are buffered: the
    buffered writes followed by the new tokens are one sequence whose
    windows start at the first buffered write (the tests compose run_windowed
    that way).
  * low-precision window buffers (variants): bf16 keys and values rounded to
    nearest even, or [PW]'s FP8 vector pairs as OCP E4M3 with one fp32
    scale absmax/448 per vector (IEEE divisions, ties to even); either way
    a token's own write enters its step exactly and is stored rounded.
  * the Pure-Write sliding window ([PW], run_sliding): the last W writes are
    kept raw, each contributing beta v k~^T with its key propagated through
    every later transition; the low-bit historical state takes every
    token's transition, absorbs each write as it leaves the window, and is
    requantized at every token (a state that changes every token is stored
    low-bit only by requantizing it); outputs come from the fp32 state
    before that requantization.

Pins (tests/test_oracle_*.py): every function below is checked against a
closed form, an invariant, a special case or a hand-derived worked example
(tests/golden/).  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# Codec  ([LQ] abstract: 8-bit recurrent state)
# --------------------------------------------------------------------------
def quantize_rows(x, qmax=127):
    """Per-row symmetric codec.  x[..., d] -> (codes int8[..., d], scale f32[...]).

    scale = max|x| / qmax (fp32 division); codes = clamp(rne(x / scale), -qmax, qmax);
    a row whose max|x| is 0 gets scale 0 and codes 0.  The decision is taken
    in fp32 whatever the input precision.  qmax = 127 is the 8-bit state;
    qmax = 7 the uniform 4-bit state ([PW]'s "@4" configuration): the same
    rule with 15 levels.
    """
    x32 = np.asarray(x).astype(F32)
    absmax = np.max(np.abs(x32), axis=-1)
    scale = (absmax / F32(qmax)).astype(F32)
    nonzero = scale > 0
    denom = np.where(nonzero, scale, F32(1.0)).astype(F32)
    ratio = (x32 / denom[..., None]).astype(F32)
    codes = np.clip(np.rint(ratio), -qmax, qmax)
    codes = np.where(nonzero[..., None], codes, 0).astype(np.int8)
    return codes, scale


def dequantize(codes, scale, dtype=F32):
    """codes * scale, row-wise, in `dtype`."""
    return np.asarray(codes).astype(dtype) * np.asarray(scale).astype(dtype)[..., None]


# --------------------------------------------------------------------------
# Walsh-Hadamard rotation  ([LIN] rotations; [BBT] WHT)
# --------------------------------------------------------------------------
def wht_matrix(d, dtype=F64):
    """Normalised Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j) / sqrt(d).

    Written out densely on purpose: the rotation is applied as a plain matrix
    product x @ H^T (H is symmetric), with no butterfly structure.
    """
    if d <= 0 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    bits = i & j
    parity = np.zeros((d, d), dtype=np.int64)
    while np.any(bits):
        parity ^= bits & 1
        bits = bits >> 1
    sign = 1 - 2 * parity
    return (sign / np.sqrt(d)).astype(dtype)


def rotate(x, dtype):
    """x[..., d] -> x @ H^T with H the normalised Sylvester matrix."""
    d = x.shape[-1]
    H = wht_matrix(d, F64).astype(dtype)
    return np.matmul(x.astype(dtype), H.T).astype(dtype)


# --------------------------------------------------------------------------
# One token of the recurrence
# --------------------------------------------------------------------------
def gdn_step(S, k, v, a, b):
    """Gated delta rule, batched over leading axes.

    S[..., dv, dk], k[..., dk], v[..., dv], a, b[...]:
        Sk = S k;   S <- a * (S - b * Sk k^T) + b * v k^T
    """
    Sk = np.matmul(S, k[..., :, None])[..., 0]
    a = a[..., None, None]
    b = b[..., None, None]
    erase = b * (Sk[..., :, None] * k[..., None, :])
    write = b * (v[..., :, None] * k[..., None, :])
    return a * (S - erase) + write


def ssd_step(S, k, v, a):
    """Scalar-decay SSD step: S <- a * S + v k^T."""
    return a[..., None, None] * S + v[..., :, None] * k[..., None, :]


# --------------------------------------------------------------------------
# The windowed algorithm ([LQ] per-window quantization; [PW] merge on exit)
# --------------------------------------------------------------------------
def _prepare_qk(q, k, rot, qk_int8, dtype, qk_bf16=False):
    q = np.asarray(q).astype(dtype)
    k = np.asarray(k).astype(dtype)
    if rot:
        q = rotate(q, dtype)
        k = rotate(k, dtype)
    if qk_bf16:
        # the rotated operands rounded to bf16, the prefill's operand precision
        q = round_bf16(q.astype(F32)).astype(dtype)
        k = round_bf16(k.astype(F32)).astype(dtype)
    if qk_int8:
        # per-token-row int8 operand quantization of the (rotated) q and k
        cq, sq = quantize_rows(q)
        ck, sk = quantize_rows(k)
        q = dequantize(cq, sq, dtype)
        k = dequantize(ck, sk, dtype)
    return q, k


def run_windowed(q, k, v, alpha, beta=None, *, W, codes0=None, scale0=None,
                 buffer0=None, kind="gdn", rot=False, qk_int8=False, dtype=F32, qmax=127,
                 qk_bf16=False):
    """Run T tokens of the windowed recurrence for N independent heads.

    q, k: [T, N, dk]; v: [T, N, dv]; alpha, beta: [T, N].
    codes0 int8 [N, dv, dk] and scale0 f32 [N, dv] give the stored low-bit
    state (None: zero state).  buffer0 = dict(k=[n0,N,dk], v=[n0,N,dv],
    alpha=[n0,N], beta=[n0,N]) holds writes already buffered in the current
    window (stored in the basis the state lives in).  W: window length, or
    None for no quantization at all (the fp reference recurrence).

    qk_bf16: the rotated q, k are rounded to bf16 (the GDN prefill's
    operand precision under the rotation).

    Steps (each one a plain reading of [LQ]/[PW]):
      1. optional rotation (then bf16 rounding or int8 operand quantization) of q, k;
      2. S = dequantize(stored codes);
      3. replay the buffered writes on top of S, oldest first;
      4. per token: S = step(S, token); o_t = S q_t; the window counter
         advances; when it reaches W the state is requantized and the
         working state restarts from the dequantized codes; otherwise the
         write joins the buffer.
    Returns dict(o [T,N,dv], codes, scale, buf dict, n, S).
    """
    q, k = _prepare_qk(q, k, rot, qk_int8, dtype, qk_bf16)
    v = np.asarray(v).astype(dtype)
    alpha = np.asarray(alpha).astype(dtype)
    beta = None if beta is None else np.asarray(beta).astype(dtype)
    T, N, dk = k.shape
    dv = v.shape[-1]

    if codes0 is None:
        codes = np.zeros((N, dv, dk), np.int8)
        scale = np.zeros((N, dv), F32)
    else:
        codes = np.array(codes0, dtype=np.int8, copy=True)
        scale = np.array(scale0, dtype=F32, copy=True)
    S = dequantize(codes, scale, dtype)

    buf = {"k": [], "v": [], "alpha": [], "beta": []}
    if buffer0 is not None:
        n0 = len(buffer0["k"])
        for i in range(n0):
            bk = np.asarray(buffer0["k"][i]).astype(dtype)
            bv = np.asarray(buffer0["v"][i]).astype(dtype)
            ba = np.asarray(buffer0["alpha"][i]).astype(dtype)
            if kind == "gdn":
                bb = np.asarray(buffer0["beta"][i]).astype(dtype)
                S = gdn_step(S, bk, bv, ba, bb)
            else:
                bb = np.zeros_like(ba)
                S = ssd_step(S, bk, bv, ba)
            buf["k"].append(bk)
            buf["v"].append(bv)
            buf["alpha"].append(ba)
            buf["beta"].append(bb)
    n = len(buf["k"])

    o = np.zeros((T, N, dv), dtype)
    for t in range(T):
        if kind == "gdn":
            S = gdn_step(S, k[t], v[t], alpha[t], beta[t])
        else:
            S = ssd_step(S, k[t], v[t], alpha[t])
        o[t] = np.matmul(S, q[t][..., :, None])[..., 0]
        n += 1
        if W is not None and n == W:
            codes, scale = quantize_rows(S, qmax)
            S = dequantize(codes, scale, dtype)
            n = 0
            buf = {"k": [], "v": [], "alpha": [], "beta": []}
        else:
            buf["k"].append(k[t])
            buf["v"].append(v[t])
            buf["alpha"].append(alpha[t])
            buf["beta"].append(beta[t] if beta is not None else np.zeros_like(alpha[t]))

    def _stack(lst, shape):
        return np.stack(lst) if lst else np.zeros((0,) + shape, dtype)

    bufs = {"k": _stack(buf["k"], (N, dk)), "v": _stack(buf["v"], (N, dv)),
            "alpha": _stack(buf["alpha"], (N,)), "beta": _stack(buf["beta"], (N,))}
    return {"o": o, "codes": codes if W is not None else None,
            "scale": scale if W is not None else None, "buf": bufs, "n": n, "S": S}


def round_bf16(x):
    """Nearest bf16 value of each fp32 entry, ties to even (finite inputs).

    bf16 keeps the top 16 bits of an fp32 word; rounding to nearest even on
    the dropped 16 bits is: add 0x7FFF plus the lowest kept bit, then clear
    the dropped bits.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=F32)).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F32)


E4M3_MAX = 448.0


def round_e4m3(x):
    """Nearest value on the OCP FP8 E4M3 grid, ties to even ([PW] keeps
    recent writes as FP8 vector pairs; the format is the common E4M3).

    E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; the largest
    finite magnitude is 448 and there is no infinity.  For |x| in
    [2^e, 2^(e+1)) with e >= -6 the grid step is 2^(e-3); below 2^-6
    (subnormals) it is 2^-9.  Rounding is rint(|x| / step) * step with
    rint ties-to-even, exact because step is a power of two.  Finite inputs
    with |x| <= 448 (larger magnitudes saturate to 448).
    """
    x = np.asarray(x, dtype=F32).astype(np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)  # a = m * 2^ex with m in [0.5, 1): e = ex - 1
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    step = np.ldexp(1.0, e - 3)
    r = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    return (np.sign(x) * r).astype(F32)


def quantize_e4m3_vector(x):
    """One FP8 E4M3 vector with one fp32 scale per vector (last axis).

    scale = absmax / 448 (an IEEE fp32 division); each entry's code is the
    E4M3 value nearest to x / scale (an IEEE fp32 division, ties to even);
    the value the buffer holds is code * scale in fp32.  An all-zero vector
    gets scale 0 and holds zeros.  Returns (values, codes as E4M3 values,
    scales).
    """
    x = np.asarray(x, dtype=F32)
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    scale = (amax / F32(E4M3_MAX)).astype(F32)
    safe = np.where(scale > 0, scale, F32(1)).astype(F32)
    c = round_e4m3((x / safe).astype(F32))
    vals = np.where(scale > 0, (c * scale).astype(F32), F32(0)).astype(F32)
    return vals, c, scale[..., 0]


def decode_step(q, k, v, alpha, beta, codes, scales, buf_k, buf_v, buf_alpha,
                buf_beta, fill, W, rot=False, dtype=F32, buf_bf16=False, buf_fp8=False, qmax=127):
    """One decode token for a batch of sequences ([LQ] per-window quantization).

    q, k: [B,H,dk]; v: [B,H,dv]; alpha, beta: [B,H]; codes [B,H,dv,dk];
    scales [B,H,dv]; buf_k [B,H,W,dk]; buf_v [B,H,W,dv]; buf_alpha,
    buf_beta [B,H,W]; fill [B] = writes already buffered for the sequence.
    With rot, q and k are rotated before use; buffered keys are already in
    the rotated basis.

    buf_bf16 (the low-precision window buffer, a variant the pages list as a
    storage option, not their default): the buffered keys and values are
    kept as bf16.  The token's own write enters this step exactly; the copy
    appended to the buffer is rounded to bf16 (round_bf16), so later steps
    and the window's close replay the rounded write.  Alpha and beta stay
    fp32.  With bf16 inputs and no rotation this is lossless.

    buf_fp8 (the pages' FP8 vector pairs, [PW]): likewise, but the appended
    key and value are each stored as an E4M3 vector with one fp32 scale
    (quantize_e4m3_vector); the buffer arrays returned here hold the values
    code * scale.

    Returns (o, codes_out, scales_out, buf_k, buf_v, buf_alpha, buf_beta,
    fill_out).  The buffer slot `fill` receives the token's write unless its
    window closes; then the sequence's codes and scales are rewritten and
    fill_out is 0 (buffer contents at slots >= fill_out are unspecified).
    """
    B, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    o = np.zeros((B, H, dv), dtype)
    codes_out = np.array(codes, copy=True)
    scales_out = np.array(scales, copy=True)
    bk_out = np.array(buf_k, dtype=F32, copy=True)
    bv_out = np.array(buf_v, dtype=F32, copy=True)
    ba_out = np.array(buf_alpha, dtype=F32, copy=True)
    bb_out = np.array(buf_beta, dtype=F32, copy=True)
    fill = np.asarray(fill)
    fill_out = np.zeros_like(fill)
    for f in np.unique(fill):
        f = int(f)
        seqs = np.nonzero(fill == f)[0]
        nh = len(seqs) * H
        buffer0 = {
            "k": np.transpose(np.asarray(buf_k)[seqs][:, :, :f], (2, 0, 1, 3)).reshape(f, nh, dk),
            "v": np.transpose(np.asarray(buf_v)[seqs][:, :, :f], (2, 0, 1, 3)).reshape(f, nh, dv),
            "alpha": np.transpose(np.asarray(buf_alpha)[seqs][:, :, :f], (2, 0, 1)).reshape(f, nh),
            "beta": np.transpose(np.asarray(buf_beta)[seqs][:, :, :f], (2, 0, 1)).reshape(f, nh),
        }
        r = run_windowed(
            np.asarray(q)[seqs].reshape(1, -1, dk), np.asarray(k)[seqs].reshape(1, -1, dk),
            np.asarray(v)[seqs].reshape(1, -1, dv), np.asarray(alpha)[seqs].reshape(1, -1),
            np.asarray(beta)[seqs].reshape(1, -1), W=W,
            codes0=np.asarray(codes)[seqs].reshape(-1, dv, dk),
            scale0=np.asarray(scales)[seqs].reshape(-1, dv),
            buffer0=buffer0, kind="gdn", rot=rot, dtype=dtype, qmax=qmax)
        nb = len(seqs)
        o[seqs] = r["o"][0].reshape(nb, H, dv)
        codes_out[seqs] = r["codes"].reshape(nb, H, dv, dk)
        scales_out[seqs] = r["scale"].reshape(nb, H, dv)
        fill_out[seqs] = r["n"]
        if r["n"] > 0:
            slot = r["n"] - 1
            wk = r["buf"]["k"][slot].reshape(nb, H, dk)
            wv = r["buf"]["v"][slot].reshape(nb, H, dv)
            if buf_bf16:
                wk, wv = round_bf16(wk), round_bf16(wv)
            elif buf_fp8:
                wk, wv = quantize_e4m3_vector(wk)[0], quantize_e4m3_vector(wv)[0]
            bk_out[seqs, :, slot] = wk
            bv_out[seqs, :, slot] = wv
            ba_out[seqs, :, slot] = r["buf"]["alpha"][slot].reshape(nb, H)
            bb_out[seqs, :, slot] = r["buf"]["beta"][slot].reshape(nb, H)
    return o, codes_out, scales_out, bk_out, bv_out, ba_out, bb_out, fill_out


def prefill(q, k, v, alpha, beta=None, *, W, kind="gdn", rot=False, qk_int8=False,
            codes0=None, scale0=None, dtype=F32, qmax=127, qk_bf16=False):
    """Prefill of a batch from a stored (or zero) state, token by token.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; alpha, beta: [B,T,H].
    Returns dict(o [B,T,H,dv], codes [B,H,dv,dk] | None, scale [B,H,dv] | None,
    S [B,H,dv,dk] working fp state, n, buf) -- buf arrays are [B,H,n,...].
    """
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]

    def tn(x):  # [B,T,H,...] -> [T, B*H, ...]
        x = np.asarray(x)
        x = np.moveaxis(x, 1, 0)
        return x.reshape((T, B * H) + x.shape[3:])

    r = run_windowed(tn(q), tn(k), tn(v), tn(alpha), None if beta is None else tn(beta),
                     W=W, kind=kind, rot=rot, qk_int8=qk_int8, qk_bf16=qk_bf16,
                     codes0=None if codes0 is None else np.asarray(codes0).reshape(B * H, dv, dk),
                     scale0=None if scale0 is None else np.asarray(scale0).reshape(B * H, dv),
                     dtype=dtype, qmax=qmax)
    o = np.moveaxis(r["o"].reshape(T, B, H, dv), 0, 1)
    out = {"o": o, "n": r["n"], "S": r["S"].reshape(B, H, dv, dk)}
    out["codes"] = None if r["codes"] is None else r["codes"].reshape(B, H, dv, dk)
    out["scale"] = None if r["scale"] is None else r["scale"].reshape(B, H, dv)
    n = r["n"]
    out["buf"] = {
        "k": np.moveaxis(r["buf"]["k"].reshape(n, B, H, dk), 0, 2),
        "v": np.moveaxis(r["buf"]["v"].reshape(n, B, H, dv), 0, 2),
        "alpha": np.moveaxis(r["buf"]["alpha"].reshape(n, B, H), 0, 2),
        "beta": np.moveaxis(r["buf"]["beta"].reshape(n, B, H), 0, 2),
    }
    return out


# --------------------------------------------------------------------------
# Pure-Write sliding window ([PW])
# --------------------------------------------------------------------------
def gdn_transition(X, k, a, b):
    """Rows X[..., m, dk] through one token's transition, without its write:
    X <- a (X - b (X k) k^T), i.e. X A with A = a (I - b k k^T).  A is
    symmetric, so a key x[..., dk] propagates as A x = the same map on the
    row x^T (pass x[..., None, :])."""
    Xk = np.matmul(X, k[..., :, None])[..., 0]
    erase = b[..., None, None] * (Xk[..., :, None] * k[..., None, :])
    return a[..., None, None] * (X - erase)


def propagate_key(x, k, a, b):
    """A key x[..., dk] through one token's transition: A x = a (x - b (k . x) k)."""
    kx = np.sum(k * x, axis=-1)
    return a[..., None] * (x - b[..., None] * kx[..., None] * k)


def run_sliding(q, k, v, alpha, beta, *, W, codes0=None, scale0=None, window0=None,
                dtype=F32, qmax=127):
    """T tokens of the Pure-Write sliding window for N heads ([PW]: recent
    pure writes are kept apart, propagated through the full GDN transition,
    and merged into the low-bit historical state once they leave the window).

    q, k: [T, N, dk]; v: [T, N, dv]; alpha, beta: [T, N].  The state is a
    low-bit historical part H (codes0 / scale0, None = zero) plus a window
    of at most W pure writes beta_i v_i k_i^T, each carried with its key
    propagated through every later transition.  window0 = dict(k, v, alpha,
    beta) of [n0, N, ...] holds the raw writes already in the window, oldest
    first (n0 <= W).  W = None: no write ever leaves; W = 0: a write merges
    at once.

    Per token t, in this order:
      1. H = dequantize(codes); H <- H A_t (every row takes the transition);
      2. every window key takes the transition, k~ <- A_t k~;
      3. the token's write joins the window with its own key (a write does
         not take its own token's transition);
      4. while the window holds more than W writes, the oldest leaves:
         H <- H + beta v k~^T;
      5. S = H + sum over the window (oldest first) of beta v k~^T;
         o_t = S q_t (the fp32 state, before the requantization);
      6. codes, scale = quantize(H): the historical state is requantized at
         every token.
    Returns dict(o [T,N,dv], codes, scale, window (raw writes oldest first),
    n (writes in the window), S (fp32 state at the last token))."""
    q = np.asarray(q).astype(dtype)
    k = np.asarray(k).astype(dtype)
    v = np.asarray(v).astype(dtype)
    alpha = np.asarray(alpha).astype(dtype)
    beta = np.asarray(beta).astype(dtype)
    T, N, dk = k.shape
    dv = v.shape[-1]
    if codes0 is None:
        codes = np.zeros((N, dv, dk), np.int8)
        scale = np.zeros((N, dv), F32)
    else:
        codes = np.array(codes0, dtype=np.int8, copy=True)
        scale = np.array(scale0, dtype=F32, copy=True)

    # window entries: raw write (k, v, alpha, beta) and the propagated key
    win = []

    def join(kk, vv, aa, bb):
        for w in win:
            w["kt"] = propagate_key(w["kt"], kk, aa, bb)
        win.append({"k": kk, "v": vv, "alpha": aa, "beta": bb, "kt": kk.copy()})

    if window0 is not None:
        for i in range(len(window0["k"])):
            join(np.asarray(window0["k"][i]).astype(dtype), np.asarray(window0["v"][i]).astype(dtype),
                 np.asarray(window0["alpha"][i]).astype(dtype), np.asarray(window0["beta"][i]).astype(dtype))

    def outer(a_, b_):
        return a_[..., :, None] * b_[..., None, :]

    o = np.zeros((T, N, dv), dtype)
    S = dequantize(codes, scale, dtype)
    for t in range(T):
        H = dequantize(codes, scale, dtype)
        H = gdn_transition(H, k[t], alpha[t], beta[t])
        join(k[t], v[t], alpha[t], beta[t])
        while W is not None and len(win) > W:
            w = win.pop(0)
            H = H + w["beta"][:, None, None] * outer(w["v"], w["kt"])
        S = H
        for w in win:
            S = S + w["beta"][:, None, None] * outer(w["v"], w["kt"])
        o[t] = np.matmul(S, q[t][..., :, None])[..., 0]
        codes, scale = quantize_rows(H, qmax)

    def _stack(key, shape):
        return np.stack([w[key] for w in win]) if win else np.zeros((0,) + shape, dtype)

    window = {"k": _stack("k", (N, dk)), "v": _stack("v", (N, dv)), "alpha": _stack("alpha", (N,)),
              "beta": _stack("beta", (N,))}
    return {"o": o, "codes": codes, "scale": scale, "window": window, "n": len(win), "S": S}


def sliding_ring_slots(fill, W):
    """Ring buffer of the sliding window (the layout decode keeps): fill in
    [0, 2W).  Below W the window holds `fill` writes in slots 0 .. fill-1;
    from W on it is full and its oldest write sits in slot fill - W.
    Returns (slots oldest first, the slot the next write takes, fill after
    one more write)."""
    fill = int(fill)
    if fill < W:
        return list(range(fill)), fill, fill + 1
    p = fill - W
    return [(p + i) % W for i in range(W)], p, W + (p + 1) % W


def decode_step_sliding(q, k, v, alpha, beta, codes, scales, buf_k, buf_v, buf_alpha, buf_beta,
                        fill, W, dtype=F32, qmax=127):
    """One decode token per sequence of the Pure-Write sliding window ([PW]).

    Shapes as decode_step; the buffer is a ring of W raw writes per head
    (sliding_ring_slots gives their order); fill [B] in [0, 2W).  The token's
    write goes into the slot the ring names (over the write that leaves);
    the historical codes and scales are rewritten every token.
    Returns (o, codes_out, scales_out, buf_k, buf_v, buf_alpha, buf_beta,
    fill_out)."""
    B, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    o = np.zeros((B, H, dv), dtype)
    codes_out = np.array(codes, copy=True)
    scales_out = np.array(scales, copy=True)
    bufs = [np.array(x, dtype=F32, copy=True) for x in (buf_k, buf_v, buf_alpha, buf_beta)]
    fill = np.asarray(fill)
    fill_out = np.zeros_like(fill)
    for b in range(B):
        slots, nxt, fo = sliding_ring_slots(fill[b], W)
        window0 = {"k": np.asarray(buf_k)[b][:, slots].transpose(1, 0, 2),
                   "v": np.asarray(buf_v)[b][:, slots].transpose(1, 0, 2),
                   "alpha": np.asarray(buf_alpha)[b][:, slots].T,
                   "beta": np.asarray(buf_beta)[b][:, slots].T}
        r = run_sliding(np.asarray(q)[b][None], np.asarray(k)[b][None], np.asarray(v)[b][None],
                        np.asarray(alpha)[b][None], np.asarray(beta)[b][None], W=W,
                        codes0=np.asarray(codes)[b], scale0=np.asarray(scales)[b], window0=window0,
                        dtype=dtype, qmax=qmax)
        o[b] = r["o"][0]
        codes_out[b] = r["codes"]
        scales_out[b] = r["scale"]
        bufs[0][b, :, nxt] = np.asarray(k)[b]
        bufs[1][b, :, nxt] = np.asarray(v)[b]
        bufs[2][b, :, nxt] = np.asarray(alpha)[b]
        bufs[3][b, :, nxt] = np.asarray(beta)[b]
        fill_out[b] = fo
    return (o, codes_out, scales_out, *bufs, fill_out)


# --------------------------------------------------------------------------
# Chunkwise-parallel form in fp64 ([LIN]: chunkwise prefill as matmuls)
# --------------------------------------------------------------------------
def chunked_fp64(q, k, v, alpha, beta=None, *, C, W=None, kind="gdn", S0=None):
    """Single head, fp64, chunk by chunk (the UT / WY form of the delta rule).

    Within a chunk of C tokens with gamma_i = prod_{s<=i} alpha_s:
      GDN:  A_ij = beta_i (gamma_i/gamma_j) k_i.k_j  (j < i, else 0)
            (I + A) U = diag(beta) V - diag(beta*gamma) K S0^T   (solved)
      SSD:  U = V
      O   = diag(gamma) Q S0^T + (L o Q K^T) U,  L_ij = gamma_i/gamma_j (j <= i)
      S_C = gamma_C S0 + U^T diag(gamma_C / gamma) K
    With W a multiple of C, the state is requantized at every window end.
    q, k: [T, dk]; v: [T, dv]; alpha, beta: [T].  Returns dict(o, S, codes, scale).
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    alpha = np.asarray(alpha, F64)
    T, dk = k.shape
    dv = v.shape[1]
    if T % C:
        raise ValueError("T must be a multiple of C")
    if W is not None and W % C:
        raise ValueError("W must be a multiple of C")
    S = np.zeros((dv, dk)) if S0 is None else np.asarray(S0, F64).copy()
    codes = scale = None
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, c0 + C)
        Qc, Kc, Vc, ac = q[sl], k[sl], v[sl], alpha[sl]
        gamma = np.cumprod(ac)
        ratio = gamma[:, None] / gamma[None, :]
        if kind == "gdn":
            bc = np.asarray(beta, F64)[sl]
            A = np.tril(bc[:, None] * ratio * (Kc @ Kc.T), -1)
            rhs = bc[:, None] * Vc - (bc * gamma)[:, None] * (Kc @ S.T)
            U = np.linalg.solve(np.eye(C) + A, rhs)
        else:
            U = Vc
        Lmask = np.tril(ratio)
        o[sl] = gamma[:, None] * (Qc @ S.T) + (Lmask * (Qc @ Kc.T)) @ U
        S = gamma[-1] * S + U.T @ ((gamma[-1] / gamma)[:, None] * Kc)
        if W is not None and (c0 + C) % W == 0:
            codes, scale = quantize_rows(S)
            S = dequantize(codes, scale, F64)
    return {"o": o, "S": S, "codes": codes, "scale": scale}


def ssd_closed_form(q, k, v, a, S0=None):
    """Quadratic ("attention") form of the scalar-decay recurrence, fp64:
    o_t = (prod_{r<=t} a_r) S0 q_t + sum_{s<=t} (prod_{r=s+1..t} a_r)(q_t.k_s) v_s.
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    a = np.asarray(a, F64)
    T, dk = k.shape
    dv = v.shape[1]
    o = np.zeros((T, dv))
    for t in range(T):
        acc = np.zeros(dv)
        if S0 is not None:
            acc += np.prod(a[: t + 1]) * (np.asarray(S0, F64) @ q[t])
        for s in range(t + 1):
            acc += np.prod(a[s + 1: t + 1]) * (q[t] @ k[s]) * v[s]
        o[t] = acc
    return o


# --------------------------------------------------------------------------
# Backward sweep (design check of the decode algorithm; not the oracle)
# --------------------------------------------------------------------------
def sweep_mirror(q, k, v, alpha, beta, codes, scale, buf_k, buf_v, buf_alpha, buf_beta,
                 dtype=F64):
    """Output of one decode token by the backward sweep, single head.

    With A_j = alpha_j (I - beta_j k_j k_j^T) (symmetric), o = S_t q unrolls to
        o = S_0 y_0 + sum_j beta_j (k_j . y_j) v_j,   y_t = q,  y_{j-1} = A_j y_j,
    where j runs over the buffered writes and the current one.  Used only to
    check that this rearrangement equals the replay; never as the reference.
    q, k: [dk]; v: [dv]; codes [dv,dk]; buf_*: [f, ...].
    """
    ks = list(np.asarray(buf_k, dtype)) + [np.asarray(k, dtype)]
    vs = list(np.asarray(buf_v, dtype)) + [np.asarray(v, dtype)]
    als = list(np.asarray(buf_alpha, dtype)) + [dtype(alpha)]
    bes = list(np.asarray(buf_beta, dtype)) + [dtype(beta)]
    y = np.asarray(q, dtype).copy()
    o = np.zeros(len(vs[0]), dtype)
    for j in range(len(ks) - 1, -1, -1):
        d = ks[j] @ y
        c = bes[j] * d
        o += c * vs[j]
        y = als[j] * (y - c * ks[j])
    return o + dequantize(codes, scale, dtype) @ y
