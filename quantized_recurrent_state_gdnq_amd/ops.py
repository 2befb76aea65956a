"""Torch-facing wrappers around the C ABI (include/gdnq.h).

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's gfx950 kernels.  These functions only check
dtype/device/contiguity, allocate outputs the caller did not pass, and hand
raw pointers to the library.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

_DT = {torch.float32: _lib.GDNQ_F32, torch.bfloat16: _lib.GDNQ_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, name, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t, shape, name):
    """The library sees raw pointers only: every buffer a caller passes must
    have exactly the shape the kernels address."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


_BUF_FLAGS = {torch.float32: 0, torch.bfloat16: _lib.GDNQ_FLAG_BUF_BF16,
              torch.float8_e4m3fn: _lib.GDNQ_FLAG_BUF_FP8}


def _state_shapes(st, B, H, d_k, d_v, window, wht=False):
    """A DecodeState handed to a prefill entry point: a window buffer of
    `window` slots (fp32, bf16 or FP8 vector pairs), codes/scales/fill of B
    sequences, rotated (keys and state in the rotated basis) exactly when
    `wht`.  Returns the window-buffer format flag."""
    if st.buf_k.dtype not in _BUF_FLAGS or st.buf_v.dtype != st.buf_k.dtype:
        raise ValueError("state: window buffers of fp32, bf16 or float8_e4m3fn (both alike)")
    if getattr(st, "sliding", False):
        raise ValueError("state: the prefill hand-over fills a tumbling window, not a sliding one")
    if bool(st.wht) != bool(wht):
        raise ValueError("state: its rotation (wht) must match the prefill's")
    if st.window != window:
        raise ValueError(f"state: window {st.window}, the prefill hand-over needs {window}")
    _shape(st.codes, (B, H, d_v, d_k * st.state_bits // 8), "state.codes")
    _shape(st.scales, (B, H, d_v), "state.scales")
    _shape(st.buf_k, (B, H, window, d_k), "state.buf_k")
    _shape(st.buf_v, (B, H, window, d_v), "state.buf_v")
    _shape(st.buf_alpha, (B, H, window), "state.buf_alpha")
    _shape(st.buf_beta, (B, H, window), "state.buf_beta")
    _shape(st.fill, (B,), "state.fill")
    return _BUF_FLAGS[st.buf_k.dtype]


def quantize_state(S, codes=None, scales=None, wht=False, state_bits=8):
    """Per-row codec of S[..., d_k] (fp32): returns (codes, scales fp32[...]).
    state_bits 8: int8 codes [..., d_k]; 4: packed 4-bit codes [..., d_k/2]
    (two per byte, column 2j in the low nibble)."""
    _need(S, "S", torch.float32)
    if state_bits not in (8, 4):
        raise ValueError("state_bits must be 8 or 4")
    d_k = S.shape[-1]
    rows = S.numel() // d_k if d_k else 0
    cshape = S.shape[:-1] + (d_k * state_bits // 8,)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.int8, device=S.device)
    if scales is None:
        scales = torch.empty(S.shape[:-1], dtype=torch.float32, device=S.device)
    _need(codes, "codes", torch.int8, S.device)
    _need(scales, "scales", torch.float32, S.device)
    if codes.shape != cshape or scales.numel() != rows:
        raise ValueError("codes must match S (packed for 4 bits); scales must hold one value per row")
    flags = (_lib.GDNQ_FLAG_WHT if wht else 0) | (_lib.GDNQ_FLAG_STATE_4BIT if state_bits == 4 else 0)
    _lib.check(_lib.quantize_state(_ptr(S), rows, d_k, _ptr(codes), _ptr(scales), flags,
                                   _stream(S.device)))
    return codes, scales


def decode_step(q, k, v, alpha, beta, codes, scales, buf_k, buf_v, buf_alpha, buf_beta,
                fill_in, fill_out, o=None, *, wht=False, out_dtype=None, sliding=False, _bind_only=False):
    """One decode token per sequence (see gdnq_decode_step in include/gdnq.h).

    q, k [B,H,d_k], v [B,H,d_v] (fp32 or bf16); alpha, beta [B,H] fp32;
    codes [B,H,d_v,d_k] int8 and scales [B,H,d_v] fp32 (updated in place for
    sequences whose window closes); buf_k [B,H,W,d_k], buf_v [B,H,W,d_v]
    (both fp32, or both bf16 for the low-precision window buffer),
    buf_alpha, buf_beta [B,H,W] fp32 (slot fill_in[b] receives the write);
    fill_in, fill_out [B] int32 (distinct).  Returns o [B,H,d_v].

    FP8 window buffer: buf_k, buf_v of dtype float8_e4m3fn, [B,H,W,d] views
    at the start of buffers that continue with the per-vector fp32 scales
    [B,H,W] (fp8_window_buffer() makes such a pair).

    4-bit state: codes [B,H,d_v,d_k/2] int8 holding packed 4-bit codes
    (inferred from the shape).

    sliding=True: the Pure-Write sliding window (GDNQ_FLAG_SLIDING): the
    buffer is a ring of the last W raw writes, fill in [0, 2W), and codes /
    scales (the historical state) are rewritten at every token.
    """
    dev = q.device
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    W = buf_k.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, dev)
    for name, t in (("alpha", alpha), ("beta", beta), ("scales", scales),
                    ("buf_alpha", buf_alpha), ("buf_beta", buf_beta)):
        _need(t, name, torch.float32, dev)
    if buf_k.dtype not in (torch.float32, torch.bfloat16, torch.float8_e4m3fn):
        raise ValueError("buf_k must be float32, bfloat16 or float8_e4m3fn")
    _need(buf_k, "buf_k", buf_k.dtype, dev)
    _need(buf_v, "buf_v", buf_k.dtype, dev)
    buf_bf16 = buf_k.dtype == torch.bfloat16
    buf_fp8 = buf_k.dtype == torch.float8_e4m3fn
    if buf_fp8:
        for name, t in (("buf_k", buf_k), ("buf_v", buf_v)):
            need = t.numel() + 4 * (t.numel() // t.shape[-1])
            if t.storage_offset() + need > t.untyped_storage().nbytes():
                raise ValueError(f"{name}: an FP8 buffer must be followed in its allocation by "
                                 "its fp32 scales (see fp8_window_buffer)")
    _need(codes, "codes", torch.int8, dev)
    _need(fill_in, "fill_in", torch.int32, dev)
    _need(fill_out, "fill_out", torch.int32, dev)
    if q.dtype not in _DT:
        raise ValueError("q, k, v must be float32 or bfloat16")
    if o is None:
        o = torch.empty((B, H, d_v), dtype=out_dtype or q.dtype, device=dev)
    _need(o, "o", None, dev)
    if o.dtype not in _DT:
        raise ValueError("o must be float32 or bfloat16")
    if (tuple(k.shape) != (B, H, d_k) or tuple(v.shape) != (B, H, d_v)
            or tuple(codes.shape) not in ((B, H, d_v, d_k), (B, H, d_v, d_k // 2))
            or tuple(scales.shape) != (B, H, d_v)
            or tuple(buf_k.shape) != (B, H, W, d_k) or tuple(buf_v.shape) != (B, H, W, d_v)
            or tuple(buf_alpha.shape) != (B, H, W) or tuple(buf_beta.shape) != (B, H, W)
            or tuple(alpha.shape) != (B, H) or tuple(beta.shape) != (B, H)
            or fill_in.numel() != B or fill_out.numel() != B or tuple(o.shape) != (B, H, d_v)):
        raise ValueError("inconsistent decode shapes")
    p = _lib.DecodeParams(B, H, d_k, d_v, W, _DT[q.dtype], _DT[o.dtype],
                          (_lib.GDNQ_FLAG_WHT if wht else 0) | (_lib.GDNQ_FLAG_BUF_BF16 if buf_bf16 else 0)
                          | (_lib.GDNQ_FLAG_BUF_FP8 if buf_fp8 else 0)
                          | (_lib.GDNQ_FLAG_STATE_4BIT if codes.shape[-1] != d_k else 0)
                          | (_lib.GDNQ_FLAG_SLIDING if sliding else 0))
    args = (p, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(codes), _ptr(scales),
            _ptr(buf_k), _ptr(buf_v), _ptr(buf_alpha), _ptr(buf_beta), _ptr(fill_in), _ptr(fill_out),
            _ptr(o), _stream(dev))
    if _bind_only:
        return o, args
    _lib.check(_lib.decode_step(*args))
    return o


def _prefill_params(q, v, *, window, chunk, wht, ssd, int8_qk, out_dtype, state_bits=8, extra_flags=0):
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    flags = ((_lib.GDNQ_FLAG_WHT if wht else 0) | (_lib.GDNQ_FLAG_SSD if ssd else 0)
             | (_lib.GDNQ_FLAG_INT8_QK if int8_qk else 0)
             | (_lib.GDNQ_FLAG_STATE_4BIT if state_bits == 4 else 0) | extra_flags)
    return _lib.PrefillParams(B, T, H, d_k, d_v, chunk, window, _DT[q.dtype], _DT[out_dtype], flags)


def prefill_workspace_size(q, v, *, window=64, chunk=64, wht=False, ssd=False, int8_qk=False,
                           out_dtype=torch.bfloat16, no_requant=False):
    p = _prefill_params(q, v, window=window, chunk=chunk, wht=wht, ssd=ssd, int8_qk=int8_qk,
                        out_dtype=out_dtype, extra_flags=_lib.GDNQ_FLAG_NO_REQUANT if no_requant else 0)
    return int(_lib.prefill_workspace_size(p))


def prefill_chunked(q, k, v, alpha, beta=None, *, window=64, chunk=64, init_codes=None,
                    init_scales=None, wht=False, ssd=False, int8_qk=False,
                    out_dtype=torch.bfloat16, o=None, codes=None, scales=None, state_f32=None,
                    workspace=None, state_bits=8, noalloc=False, no_requant=False, state=None):
    """Chunkwise prefill (see gdnq_prefill_chunked in include/gdnq.h).

    state (a DecodeState, GDN only): its window buffer and fills take the
    open window's T mod window writes, as the hand-over does, and its codes
    and scales the state at the last window boundary (codes/scales must then
    be None); required when T is not a multiple of the window.  Returns
    (o, state.codes, state.scales).

    q, k [B,T,H,d_k], v [B,T,H,d_v] bf16; alpha (and beta for GDN) [B,T,H] fp32.
    GDN returns (o, codes, scales); SSD (ssd=True) returns (o, state_f32), and
    so does GDN with no_requant=True (GDNQ_FLAG_NO_REQUANT: the state is never
    requantized and comes back in fp32).
    GDN with state_bits=4: the uniform 4-bit state, codes [B,H,d_v,d_k/2]
    packed two per byte (init_codes likewise).
    noalloc=True calls gdnq_prefill_chunked_noalloc (the library's own device
    scratch instead of a workspace; pass o and the state outputs to keep the
    call free of allocations).
    """
    dev = q.device
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev)
    _need(alpha, "alpha", torch.float32, dev)
    if tuple(k.shape) != (B, T, H, d_k) or tuple(v.shape) != (B, T, H, d_v) or tuple(alpha.shape) != (B, T, H):
        raise ValueError("inconsistent prefill shapes")
    if state is not None or (not ssd and not no_requant and window > 0 and T % window != 0):
        if state is None:
            raise ValueError(f"T = {T} is not a multiple of the window {window}: pass state= (a DecodeState) "
                             "to receive the open window's writes")
        if ssd or no_requant or state_f32 is not None or codes is not None or scales is not None:
            raise ValueError("with state=, the state goes to state.codes/state.scales (GDN, no state_f32, "
                             "codes or scales)")
        if state.state_bits != state_bits:
            raise ValueError("state: its code width differs from state_bits")
        _need(beta, "beta", torch.float32, dev)
        if tuple(beta.shape) != (B, T, H):
            raise ValueError("beta must be [B,T,H]")
        p = _prefill_params(q, v, window=window, chunk=chunk, wht=wht, ssd=False, int8_qk=False,
                            out_dtype=out_dtype, state_bits=state_bits,
                            extra_flags=_state_shapes(state, B, H, d_k, d_v, window, wht))
        if o is None:
            o = torch.empty((B, T, H, d_v), dtype=out_dtype, device=dev)
        _shape(_need(o, "o", out_dtype, dev), (B, T, H, d_v), "o")
        _init_shapes(init_codes, init_scales, (B, H, d_v, d_k * state_bits // 8), dev)
        bufs = dict(buf_k=_ptr(state.buf_k), buf_v=_ptr(state.buf_v), buf_alpha=_ptr(state.buf_alpha),
                    buf_beta=_ptr(state.buf_beta), fill_out=_ptr(state.fill))
        args = (p, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(init_codes), _ptr(init_scales),
                _ptr(o), _ptr(state.codes), _ptr(state.scales), None)
        if noalloc:
            if workspace is not None:
                raise ValueError("noalloc: no workspace is taken")
            _lib.check(_lib.prefill_chunked_noalloc(*args, _stream(dev), **bufs))
        else:
            need = int(_lib.prefill_workspace_size(p))
            if need and workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
            _lib.check(_lib.prefill_chunked(*args, _ptr(workspace), ws_bytes, _stream(dev), **bufs))
        return o, state.codes, state.scales
    p = _prefill_params(q, v, window=window, chunk=chunk, wht=wht, ssd=ssd, int8_qk=int8_qk,
                        out_dtype=out_dtype, state_bits=state_bits,
                        extra_flags=_lib.GDNQ_FLAG_NO_REQUANT if no_requant else 0)
    if o is None:
        o = torch.empty((B, T, H, d_v), dtype=out_dtype, device=dev)
    _shape(_need(o, "o", out_dtype, dev), (B, T, H, d_v), "o")
    f32_state = ssd or no_requant  # the final state comes back in fp32
    if state_f32 is not None and not f32_state:
        raise ValueError("state_f32 is an output of SSD and no_requant calls only")
    if f32_state:
        if codes is not None or scales is not None:
            raise ValueError("codes and scales are not outputs here (the state comes back as state_f32)")
        if state_f32 is None:
            state_f32 = torch.empty((B, H, d_v, d_k), dtype=torch.float32, device=dev)
        _shape(_need(state_f32, "state_f32", torch.float32, dev), (B, H, d_v, d_k), "state_f32")
    if not ssd:
        _need(beta, "beta", torch.float32, dev)
        if tuple(beta.shape) != (B, T, H):
            raise ValueError("beta must be [B,T,H]")
        cshape = (B, H, d_v, d_k * state_bits // 8)
        if not no_requant:
            if codes is None:
                codes = torch.empty(cshape, dtype=torch.int8, device=dev)
            if scales is None:
                scales = torch.empty((B, H, d_v), dtype=torch.float32, device=dev)
            _shape(_need(codes, "codes", torch.int8, dev), cshape, "codes")
            _shape(_need(scales, "scales", torch.float32, dev), (B, H, d_v), "scales")
        if (init_codes is None) != (init_scales is None):
            raise ValueError("init_codes and init_scales: both or neither")
        if init_codes is not None:
            _shape(_need(init_codes, "init_codes", torch.int8, dev), cshape, "init_codes")
            _shape(_need(init_scales, "init_scales", torch.float32, dev), (B, H, d_v), "init_scales")
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc: no workspace is taken")
        _lib.check(_lib.prefill_chunked_noalloc(p, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                                None if ssd else _ptr(beta), _ptr(init_codes),
                                                _ptr(init_scales), _ptr(o), _ptr(codes), _ptr(scales),
                                                _ptr(state_f32), _stream(dev)))
        return (o, state_f32) if f32_state else (o, codes, scales)
    need = int(_lib.prefill_workspace_size(p))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(_lib.prefill_chunked(p, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    None if ssd else _ptr(beta), _ptr(init_codes),
                                    _ptr(init_scales), _ptr(o), _ptr(codes), _ptr(scales), _ptr(state_f32),
                                    _ptr(workspace), ws_bytes, _stream(dev)))
    if f32_state:
        return o, state_f32
    return o, codes, scales


def _init_shapes(init_codes, init_scales, cshape, dev):
    if (init_codes is None) != (init_scales is None):
        raise ValueError("init_codes and init_scales: both or neither")
    if init_codes is not None:
        _shape(_need(init_codes, "init_codes", torch.int8, dev), cshape, "init_codes")
        _shape(_need(init_scales, "init_scales", torch.float32, dev), cshape[:3], "init_scales")


def prefill_handoff_workspace_size(q, v, *, window=64, out_dtype=torch.bfloat16, wht=False, chunk=64):
    p = _prefill_params(q, v, window=window, chunk=chunk, wht=wht, ssd=False, int8_qk=False,
                        out_dtype=out_dtype)
    return int(_lib.prefill_handoff_workspace_size(p))


def prefill_handoff(q, k, v, alpha, beta, *, window=64, init_codes=None, init_scales=None,
                    out_dtype=torch.bfloat16, o=None, state=None, workspace=None, state_bits=8,
                    buf_dtype=torch.float32, wht=False, chunk=64):
    """GDN prefill of any T tokens handed over to decode (see
    gdnq_prefill_handoff in include/gdnq.h): returns (o, DecodeState) whose
    codes/scales are the state at the last window boundary and whose window
    buffer (decode's `window` of 1..64 slots; fp32, bf16 or FP8 vector pairs:
    buf_dtype, or the given state's) holds the last T mod window writes, with
    that fill; with wht=True q and k are rotated and the state and buffered
    keys are in the rotated basis.  o, state and workspace may be given to
    reuse their memory."""
    dev = q.device
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev)
    for name, t in (("alpha", alpha), ("beta", beta)):
        _need(t, name, torch.float32, dev)
    if (tuple(k.shape) != (B, T, H, d_k) or tuple(v.shape) != (B, T, H, d_v)
            or tuple(alpha.shape) != (B, T, H) or tuple(beta.shape) != (B, T, H)):
        raise ValueError("inconsistent prefill shapes")
    if o is None:
        o = torch.empty((B, T, H, d_v), dtype=out_dtype, device=dev)
    _shape(_need(o, "o", out_dtype, dev), (B, T, H, d_v), "o")
    _init_shapes(init_codes, init_scales, (B, H, d_v, d_k * state_bits // 8), dev)
    st = state
    if st is None:
        st = DecodeState(torch.empty((B, H, d_v, d_k * state_bits // 8), dtype=torch.int8, device=dev),
                         torch.empty((B, H, d_v), dtype=torch.float32, device=dev), window,
                         fill=torch.zeros(B, dtype=torch.int32, device=dev), wht=wht, state_bits=state_bits,
                         buf_dtype=buf_dtype)
    if st.state_bits != state_bits:
        raise ValueError("state: its code width differs from state_bits")
    p = _prefill_params(q, v, window=window, chunk=chunk, wht=wht, ssd=False, int8_qk=False,
                        out_dtype=out_dtype, state_bits=state_bits,
                        extra_flags=_state_shapes(st, B, H, d_k, d_v, window, wht))
    need = int(_lib.prefill_handoff_workspace_size(p))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(_lib.prefill_handoff(p, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(init_codes), _ptr(init_scales), _ptr(o), _ptr(st.codes),
                                    _ptr(st.scales), _ptr(st.buf_k), _ptr(st.buf_v),
                                    _ptr(st.buf_alpha), _ptr(st.buf_beta), _ptr(st.fill),
                                    _ptr(workspace), ws_bytes, _stream(dev)))
    return o, st


def _varlen_params(q, v, n_seqs, *, window, out_dtype, state_bits=8, extra_flags=0):
    T, H, d_k = q.shape
    return _lib.PrefillParams(n_seqs, T, H, d_k, v.shape[-1], 64, window, _DT[q.dtype],
                              _DT[out_dtype], (_lib.GDNQ_FLAG_STATE_4BIT if state_bits == 4 else 0) | extra_flags)


def prefill_varlen_workspace_size(q, v, n_seqs, *, window=64, out_dtype=torch.bfloat16, wht=False):
    p = _varlen_params(q, v, n_seqs, window=window, out_dtype=out_dtype,
                       extra_flags=_lib.GDNQ_FLAG_WHT if wht else 0)
    return int(_lib.prefill_varlen_workspace_size(p))


def prefill_varlen(q, k, v, alpha, beta, cu_seqlens, *, window=64, init_codes=None,
                   init_scales=None, out_dtype=torch.bfloat16, o=None, state=None,
                   workspace=None, state_bits=8, buf_dtype=torch.float32, wht=False):
    """GDN prefill of a packed batch of variable-length sequences handed over
    to decode (see gdnq_prefill_varlen in include/gdnq.h).  q, k [T,H,d_k],
    v [T,H,d_v] bf16 and alpha, beta [T,H] fp32 hold the sequences back to
    back; cu_seqlens (int32 on the device, B+1 entries) gives where each
    starts.  Returns (o [T,H,d_v], DecodeState of B sequences; its window
    buffer of buf_dtype, or the given state's); wht=True rotates q and k
    (state and buffered keys in the rotated basis)."""
    dev = q.device
    T, H, d_k = q.shape
    d_v = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev)
    for name, t in (("alpha", alpha), ("beta", beta)):
        _need(t, name, torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens: one dimension of B+1 offsets")
    B = cu_seqlens.numel() - 1
    if (tuple(k.shape) != (T, H, d_k) or tuple(v.shape) != (T, H, d_v)
            or tuple(alpha.shape) != (T, H) or tuple(beta.shape) != (T, H)):
        raise ValueError("inconsistent packed prefill shapes")
    if o is None:
        o = torch.empty((T, H, d_v), dtype=out_dtype, device=dev)
    _shape(_need(o, "o", out_dtype, dev), (T, H, d_v), "o")
    _init_shapes(init_codes, init_scales, (B, H, d_v, d_k * state_bits // 8), dev)
    st = state
    if st is None:
        st = DecodeState(torch.empty((B, H, d_v, d_k * state_bits // 8), dtype=torch.int8, device=dev),
                         torch.empty((B, H, d_v), dtype=torch.float32, device=dev), window,
                         fill=torch.zeros(B, dtype=torch.int32, device=dev), wht=wht, state_bits=state_bits,
                         buf_dtype=buf_dtype)
    if st.state_bits != state_bits:
        raise ValueError("state: its code width differs from state_bits")
    p = _varlen_params(q, v, B, window=window, out_dtype=out_dtype, state_bits=state_bits,
                       extra_flags=_state_shapes(st, B, H, d_k, d_v, window, wht)
                       | (_lib.GDNQ_FLAG_WHT if wht else 0))
    need = int(_lib.prefill_varlen_workspace_size(p))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(_lib.prefill_varlen(p, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(init_codes), _ptr(init_scales), _ptr(o),
                                   _ptr(st.codes), _ptr(st.scales), _ptr(st.buf_k), _ptr(st.buf_v),
                                   _ptr(st.buf_alpha), _ptr(st.buf_beta), _ptr(st.fill),
                                   _ptr(workspace), ws_bytes, _stream(dev)))
    return o, st


def prefill_resume_workspace_size(q, v, n_seqs, *, packed=False, out_dtype=torch.bfloat16, wht=False, window=64):
    """Workspace of prefill_resume: q [B,T,H,d_k] (n_seqs = B), or packed
    q [T,H,d_k] of n_seqs sequences, resuming states of decode's `window`."""
    T = q.shape[0] if packed else q.shape[1]
    p = _lib.PrefillParams(n_seqs, T, q.shape[-2], q.shape[-1], v.shape[-1], 64, window, _DT[q.dtype],
                           _DT[out_dtype], _lib.GDNQ_FLAG_WHT if wht else 0)
    return int(_lib.prefill_resume_workspace_size(p, packed))


def prefill_resume(state, q, k, v, alpha, beta, cu_seqlens=None, *, out_dtype=torch.bfloat16,
                   o=None, workspace=None):
    """Continue every sequence of a DecodeState (any window 1..64; fp32, bf16 or FP8
    window buffer, whose writes enter at bf16) with new tokens by chunked prefill, at whatever fill each sequence
    is (see gdnq_prefill_resume in include/gdnq.h).  Uniform: q, k
    [B,T,H,d_k], v [B,T,H,d_v], alpha, beta [B,T,H]; packed: [T,...] with
    cu_seqlens (int32, B+1 offsets).  Updates the state in place (codes,
    scales, buffer, fill) and returns o for the new tokens."""
    dev = q.device
    st = state
    B, H, d_v, d_k = st.codes.shape
    d_k = d_k * 8 // st.state_bits
    W = st.window
    buf_flag = _state_shapes(st, B, H, d_k, d_v, W, st.wht)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev)
    for name, t in (("alpha", alpha), ("beta", beta)):
        _need(t, name, torch.float32, dev)
    if cu_seqlens is None:
        T = q.shape[1]
        lead = (B, T)
        if q.dim() != 4 or q.shape[0] != B:
            raise ValueError("q: [B,T,H,d_k] for the state's B sequences")
    else:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() != B + 1:
            raise ValueError("cu_seqlens: B+1 offsets for the state's B sequences")
        T = q.shape[0]
        lead = (T,)
    if (tuple(q.shape) != lead + (H, d_k) or tuple(k.shape) != lead + (H, d_k)
            or tuple(v.shape) != lead + (H, d_v) or tuple(alpha.shape) != lead + (H,)
            or tuple(beta.shape) != lead + (H,)):
        raise ValueError("inconsistent resume shapes")
    p = _lib.PrefillParams(B, T, H, d_k, d_v, 64, W, _DT[q.dtype], _DT[out_dtype],
                           (_lib.GDNQ_FLAG_STATE_4BIT if st.state_bits == 4 else 0) | buf_flag
                           | (_lib.GDNQ_FLAG_WHT if st.wht else 0))
    if o is None:
        o = torch.empty(lead + (H, d_v), dtype=out_dtype, device=dev)
    _shape(_need(o, "o", out_dtype, dev), lead + (H, d_v), "o")
    need = int(_lib.prefill_resume_workspace_size(p, cu_seqlens is not None))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(_lib.prefill_resume(p, _ptr(cu_seqlens), _ptr(st.fill), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(alpha), _ptr(beta), _ptr(o), _ptr(st.codes), _ptr(st.scales),
                                   _ptr(st.buf_k), _ptr(st.buf_v), _ptr(st.buf_alpha),
                                   _ptr(st.buf_beta), _ptr(st.fill), _ptr(workspace), ws_bytes,
                                   _stream(dev)))
    return o


def fp8_window_buffer(B, H, W, d, device):
    """One FP8 window buffer: E4M3 codes [B,H,W,d] followed, in the same
    allocation, by the per-vector fp32 scales [B,H,W].  Returns (codes view,
    scales view); pass the codes view as buf_k or buf_v."""
    n = B * H * W
    raw = torch.empty(n * d + 4 * n, dtype=torch.uint8, device=device)
    codes = raw[:n * d].view(torch.float8_e4m3fn).view(B, H, W, d)
    scales = raw[n * d:].view(torch.float32).view(B, H, W)
    return codes, scales


class DecodeState:
    """Per-request state of a batch of sequences: int8 codes, per-row scales,
    the window buffer and the fill counters (ping-ponged between two arrays,
    since every head of a sequence reads the fill while the step runs)."""

    def __init__(self, codes, scales, window, fill=None, wht=False, buf_dtype=torch.float32,
                 state_bits=8, sliding=False):
        """buf_dtype: torch.float32 (the method's fp32 window buffer),
        torch.bfloat16 (writes stored rounded) or torch.float8_e4m3fn (FP8
        vector pairs: E4M3 codes with a per-vector scale, buf_k_scale and
        buf_v_scale).  state_bits 4: codes are packed 4-bit [B,H,d_v,d_k/2]."""
        B, H, d_v, d_k = codes.shape
        d_k = d_k * 8 // state_bits
        dev = codes.device
        self.codes, self.scales, self.window, self.wht = codes, scales, window, wht
        self.state_bits = state_bits
        self.sliding = sliding
        if buf_dtype == torch.float8_e4m3fn:
            self.buf_k, self.buf_k_scale = fp8_window_buffer(B, H, window, d_k, dev)
            self.buf_v, self.buf_v_scale = fp8_window_buffer(B, H, window, d_v, dev)
        else:
            self.buf_k = torch.empty((B, H, window, d_k), dtype=buf_dtype, device=dev)
            self.buf_v = torch.empty((B, H, window, d_v), dtype=buf_dtype, device=dev)
        self.buf_alpha = torch.empty((B, H, window), dtype=torch.float32, device=dev)
        self.buf_beta = torch.empty((B, H, window), dtype=torch.float32, device=dev)
        self.fill = torch.zeros(B, dtype=torch.int32, device=dev) if fill is None else fill
        self._fill_next = torch.empty_like(self.fill)

    def bind(self, q, k, v, alpha, beta, o):
        """Validate once for token buffers that are reused every step (a
        serving loop writes each new token into them) and return a
        zero-argument callable that launches one step on the current stream
        and advances the fill ping-pong."""
        _, a0 = decode_step(q, k, v, alpha, beta, self.codes, self.scales, self.buf_k, self.buf_v,
                            self.buf_alpha, self.buf_beta, self.fill, self._fill_next, o,
                            wht=self.wht, sliding=self.sliding, _bind_only=True)
        _, a1 = decode_step(q, k, v, alpha, beta, self.codes, self.scales, self.buf_k, self.buf_v,
                            self.buf_alpha, self.buf_beta, self._fill_next, self.fill, o,
                            wht=self.wht, sliding=self.sliding, _bind_only=True)
        f0 = self.fill
        orient = [(ctypes.byref(a[0]),) + tuple(a[1:]) for a in (a0, a1)]
        fn = _lib.lib.gdnq_decode_step

        def launch():
            st = fn(*orient[0 if self.fill is f0 else 1])
            if st:
                _lib.check(st)
            self.fill, self._fill_next = self._fill_next, self.fill
        return launch

    def step(self, q, k, v, alpha, beta, o=None, out_dtype=None):
        o = decode_step(q, k, v, alpha, beta, self.codes, self.scales, self.buf_k, self.buf_v,
                        self.buf_alpha, self.buf_beta, self.fill, self._fill_next, o,
                        wht=self.wht, out_dtype=out_dtype, sliding=self.sliding)
        self.fill, self._fill_next = self._fill_next, self.fill
        return o
