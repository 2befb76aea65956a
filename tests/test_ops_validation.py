"""Shape checks of the torch wrappers.  The C ABI sees raw pointers only, so
the wrappers must refuse any buffer whose shape differs from what the kernels
address (a short output, a 4-bit-sized code array on the 8-bit path, a
decode state whose window or width is not the call's) before anything is
launched.

The CPU tests call the checking helpers on host tensors; the GPU tests call
each prefill wrapper with one mis-shaped buffer and expect ValueError."""

import numpy as np
import pytest
import torch

from quantized_recurrent_state_gdnq_amd import ops


def _state(B=2, H=2, d=128, W=64, bits=8, device="cpu"):
    codes = torch.zeros((B, H, d, d * bits // 8), dtype=torch.int8, device=device)
    scales = torch.zeros((B, H, d), dtype=torch.float32, device=device)
    return ops.DecodeState(codes, scales, W, state_bits=bits)


def test_shape_helper():
    t = torch.zeros((2, 3, 4))
    assert ops._shape(t, (2, 3, 4), "t") is t
    with pytest.raises(ValueError, match="t must have shape"):
        ops._shape(t, (2, 3, 5), "t")


def test_state_shapes_accepts_matching_state():
    ops._state_shapes(_state(), 2, 2, 128, 128, 64)
    ops._state_shapes(_state(bits=4), 2, 2, 128, 128, 64)


@pytest.mark.parametrize("kw,args", [
    (dict(W=16), (2, 2, 128, 128, 64)),          # window 16: the hand-over strides 64 slots
    (dict(B=1), (2, 2, 128, 128, 64)),           # fewer sequences than the call
    (dict(H=3), (2, 2, 128, 128, 64)),
    (dict(d=64), (2, 2, 128, 128, 64)),
])
def test_state_shapes_rejects(kw, args):
    with pytest.raises(ValueError):
        ops._state_shapes(_state(**kw), *args)


def test_state_shapes_buffer_formats():
    """The hand-over takes decode's fp32, bf16 and FP8 window buffers (the
    format flag it returns goes into the call), not a rotated or a sliding
    state, nor key and value buffers of different types."""
    codes = torch.zeros((2, 2, 128, 128), dtype=torch.int8)
    for dt, flag in ((torch.float32, 0), (torch.bfloat16, 16), (torch.float8_e4m3fn, 32)):
        st = ops.DecodeState(codes, torch.zeros((2, 2, 128)), 64, buf_dtype=dt)
        assert ops._state_shapes(st, 2, 2, 128, 128, 64) == flag
    st = ops.DecodeState(codes, torch.zeros((2, 2, 128)), 64, buf_dtype=torch.bfloat16)
    st.buf_v = torch.zeros((2, 2, 64, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="both alike"):
        ops._state_shapes(st, 2, 2, 128, 128, 64)
    with pytest.raises(ValueError, match="rotation"):
        ops._state_shapes(ops.DecodeState(codes, torch.zeros((2, 2, 128)), 64, wht=True), 2, 2, 128, 128, 64)
    with pytest.raises(ValueError, match="sliding"):
        ops._state_shapes(ops.DecodeState(codes, torch.zeros((2, 2, 128)), 64, sliding=True), 2, 2, 128, 128, 64)


gpu = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _prefill_inputs(B=1, T=64, H=2, d=128, packed=False):
    dev = _dev()
    lead = (T,) if packed else (B, T)
    q = torch.zeros(lead + (H, d), dtype=torch.bfloat16, device=dev)
    a = torch.ones(lead + (H,), dtype=torch.float32, device=dev)
    return q, q.clone(), q.clone(), a, a.clone()


@gpu
@pytest.mark.parametrize("what", ["o", "codes", "scales", "init_codes", "init_scales"])
def test_prefill_chunked_rejects_misshaped(what):
    dev = _dev()
    q, k, v, a, b = _prefill_inputs()
    kw = dict(o=torch.empty((1, 64, 2, 128), dtype=torch.bfloat16, device=dev),
              codes=torch.empty((1, 2, 128, 128), dtype=torch.int8, device=dev),
              scales=torch.empty((1, 2, 128), dtype=torch.float32, device=dev),
              init_codes=torch.zeros((1, 2, 128, 128), dtype=torch.int8, device=dev),
              init_scales=torch.zeros((1, 2, 128), dtype=torch.float32, device=dev))
    bad = {"o": (1, 63, 2, 128), "codes": (1, 2, 128, 64), "scales": (1, 2, 64),
           "init_codes": (1, 2, 128, 64), "init_scales": (2, 128)}[what]
    kw[what] = torch.zeros(bad, dtype=kw[what].dtype, device=dev)
    with pytest.raises(ValueError):
        ops.prefill_chunked(q, k, v, a, b, **kw)


@gpu
def test_prefill_ssd_rejects_misshaped_state():
    dev = _dev()
    q, k, _, a, _ = _prefill_inputs()
    v = torch.zeros((1, 64, 2, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        ops.prefill_chunked(q, k, v, a, None, ssd=True, int8_qk=True,
                            state_f32=torch.empty((1, 2, 128, 128), dtype=torch.float32, device=dev))


@gpu
@pytest.mark.parametrize("what", ["o", "window16", "init_codes", "state_bits"])
def test_prefill_handoff_rejects_misshaped(what):
    dev = _dev()
    q, k, v, a, b = _prefill_inputs(T=37)
    kw = {}
    if what == "o":
        kw["o"] = torch.empty((1, 36, 2, 128), dtype=torch.bfloat16, device=dev)
    elif what == "window16":
        kw["state"] = _state(B=1, W=16, device=dev)
    elif what == "init_codes":
        kw["init_codes"] = torch.zeros((1, 2, 128, 64), dtype=torch.int8, device=dev)
        kw["init_scales"] = torch.zeros((1, 2, 128), dtype=torch.float32, device=dev)
    else:
        kw["state"] = _state(B=1, bits=4, device=dev)  # a 4-bit state on the 8-bit call
    with pytest.raises(ValueError):
        ops.prefill_handoff(q, k, v, a, b, **kw)


@gpu
@pytest.mark.parametrize("what", ["o", "window16", "nseq"])
def test_prefill_varlen_rejects_misshaped(what):
    dev = _dev()
    q, k, v, a, b = _prefill_inputs(T=100, packed=True)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device=dev)
    kw = {}
    if what == "o":
        kw["o"] = torch.empty((99, 2, 128), dtype=torch.bfloat16, device=dev)
    elif what == "window16":
        kw["state"] = _state(B=2, W=16, device=dev)
    else:
        kw["state"] = _state(B=3, device=dev)
    with pytest.raises(ValueError):
        ops.prefill_varlen(q, k, v, a, b, cu, **kw)


@gpu
@pytest.mark.parametrize("what", ["o", "d64_state"])
def test_prefill_resume_rejects_misshaped(what):
    dev = _dev()
    q, k, v, a, b = _prefill_inputs(B=2, T=10)
    st = _state(B=2, d=64 if what == "d64_state" else 128, device=dev)  # a d = 64 state for d = 128 tokens
    kw = {}
    if what == "o":
        kw["o"] = torch.empty((2, 10, 2, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        ops.prefill_resume(st, q, k, v, a, b, **kw)
