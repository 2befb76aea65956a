"""GPU parity of the prefill hand-over to decode (gdnq_prefill_handoff):
GDN prefill of any number of tokens, its open window left in decode's fp32
window buffer, then decode steps that continue the sequence.  The oracle is
the same token-by-token windowed recurrence (its state after T tokens: the
codes of the last window boundary plus the T mod 64 buffered writes).

Bars as in the prefill tests: o within 1e-3 (fp32 output) of the oracle;
codes +-1 on <= 0.1% and scales 1e-5 where the oracle starts from the same
state; free-running scales within 2/127; buffered writes bitwise (bf16
inputs are exact in fp32).
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (assert_free_scales, DEV, OUT_TOL_BF16, OUT_TOL_F32, assert_codes, assert_scales, dev, host,
                      max_rel_err)

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops

W = 64


def _inputs(x):
    return (dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
            dev(x["alpha"]), dev(x["beta"]))


def _random_state(B, H, d, seed):
    g = np.random.default_rng(seed)
    S = (g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    return O.quantize_rows(S)


def _check(st, o, ref, T, tol, teacher_codes):
    r = T % W
    if T:
        err = max_rel_err(host(o), ref["o"])
        assert err <= tol, f"o max relative error {err:.3e}"
    assert np.all(host(st.fill) == r)
    if teacher_codes:
        assert_codes(host(st.codes), ref["codes"], "codes at the last boundary")
        assert_scales(host(st.scales), ref["scale"], "scales at the last boundary")
    else:
        assert_codes(host(st.codes), ref["codes"], "codes at the last boundary")
        assert_free_scales(host(st.scales), ref["scale"], "hand-over scales at the last boundary")
    for name, key in (("buf_k", "k"), ("buf_v", "v"), ("buf_alpha", "alpha"), ("buf_beta", "beta")):
        assert np.array_equal(host(getattr(st, name))[:, :, :r], ref["buf"][key]), name


@pytest.mark.parametrize("T", [0, 1, 37, 63, 64, 65, 100, 191])
def test_handoff_matches_oracle(T):
    """B=2, H=3 from a stored state, T tokens in one call (up to two window
    closes and a partial window): outputs, the boundary state and the
    buffered writes against the oracle."""
    B, H, d = 2, 3, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T + 1)
    codes, scales = _random_state(B, H, d, T + 2)
    o, st = ops.prefill_handoff(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales),
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    assert ref["n"] == T % W
    _check(st, o, ref, T, OUT_TOL_F32 if T < 64 else OUT_TOL_BF16, teacher_codes=T < 128)


def test_handoff_whole_windows_equal_chunked_prefill():
    """T a multiple of 64: the hand-over gives the chunked prefill's outputs
    and state bitwise, with an empty buffer (fill 0)."""
    B, H, d, T = 2, 2, 128, 192
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=5)
    a_o, a_c, a_s = ops.prefill_chunked(*_inputs(x), out_dtype=torch.float32)
    b_o, st = ops.prefill_handoff(*_inputs(x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_c, st.codes) and torch.equal(a_s, st.scales)
    assert not host(st.fill).any()


@pytest.mark.parametrize("T", [37, 100])
def test_handoff_then_decode_continues(T):
    """Prefill T tokens with the hand-over, then 80 decode steps on the
    GPU's DecodeState (crossing at least one window close), against the
    oracle continuing from its own prefill state: each step teacher-forced
    (the oracle starts from the GPU's state before the step) and the outputs
    free-running."""
    B, H, d, steps = 2, 2, 128, 80
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T + 11)
    o, st = ops.prefill_handoff(*_inputs(x), out_dtype=torch.float32)
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W)
    fill = np.full(B, ref["n"], np.int32)
    bk = np.zeros((B, H, W, d), np.float32)
    bv = np.zeros((B, H, W, d), np.float32)
    ba = np.zeros((B, H, W), np.float32)
    bb = np.zeros((B, H, W), np.float32)
    n = ref["n"]
    bk[:, :, :n], bv[:, :, :n] = ref["buf"]["k"], ref["buf"]["v"]
    ba[:, :, :n], bb[:, :, :n] = ref["buf"]["alpha"], ref["buf"]["beta"]
    fr = [ref["codes"], ref["scale"], bk, bv, ba, bb, fill]
    worst_tf = worst_fr = 0.0
    n_close = 0
    for t in range(steps):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=T + 12)
        before = [host(z).copy() for z in (st.codes, st.scales, st.buf_k, st.buf_v, st.buf_alpha,
                                           st.buf_beta, st.fill)]
        go = host(st.step(dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16),
                          dev(y["v"], torch.bfloat16), dev(y["alpha"]), dev(y["beta"]),
                          out_dtype=torch.float32))
        ro, rc, rs, *_ = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *before, W)
        worst_tf = max(worst_tf, max_rel_err(go, ro))
        closing = before[6] + 1 == W
        if closing.any():
            n_close += 1
            assert_codes(host(st.codes)[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
        fo, *fr = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *fr, W)
        worst_fr = max(worst_fr, max_rel_err(go, fo))
    assert n_close >= 1
    assert worst_tf <= OUT_TOL_BF16, worst_tf
    assert worst_fr <= OUT_TOL_BF16, worst_fr


def test_handoff_larger_batch():
    """B=4, H=8, T=1000 (15 windows and 40 open writes) against the oracle
    run on its own."""
    B, H, d, T = 4, 8, 128, 1000
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=21)
    o, st = ops.prefill_handoff(*_inputs(x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W)
    _check(st, o, ref, T, OUT_TOL_BF16, teacher_codes=False)


STATE = ("codes", "scales", "buf_k", "buf_v", "buf_alpha", "buf_beta", "fill")


def _fresh(B, H, d, window, buf_dtype=torch.float32):
    return ops.DecodeState(torch.empty((B, H, d, d), dtype=torch.int8, device=DEV),
                           torch.empty((B, H, d), dtype=torch.float32, device=DEV), window,
                           fill=torch.zeros(B, dtype=torch.int32, device=DEV), buf_dtype=buf_dtype)


@pytest.mark.parametrize("T,window,buf", [(100, 64, torch.float32), (37, 16, torch.bfloat16),
                                          (90, 64, torch.float8_e4m3fn)])
def test_chunked_with_window_buffer_is_the_handoff(T, window, buf):
    """gdnq_prefill_chunked given decode's window buffer (T not a multiple
    of the window) gives bitwise the results of gdnq_prefill_handoff, with
    a workspace and through the allocation-free entry point."""
    B, H, d = 2, 3, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=200 + T)
    c0, s0 = _random_state(B, H, d, 201)
    args = _inputs(x)
    o1, st1 = ops.prefill_handoff(*args, window=window, init_codes=dev(c0), init_scales=dev(s0),
                                  out_dtype=torch.float32, buf_dtype=buf)
    st2 = _fresh(B, H, d, window, buf)
    o2, c2, s2 = ops.prefill_chunked(*args, window=window, init_codes=dev(c0), init_scales=dev(s0),
                                     out_dtype=torch.float32, state=st2)
    st3 = _fresh(B, H, d, window, buf)
    o3, _, _ = ops.prefill_chunked(*args, window=window, init_codes=dev(c0), init_scales=dev(s0),
                                   out_dtype=torch.float32, state=st3, noalloc=True)
    torch.cuda.synchronize()
    assert c2 is st2.codes and s2 is st2.scales
    r = T % window
    names = STATE + (("buf_k_scale", "buf_v_scale") if buf == torch.float8_e4m3fn else ())
    for o, st, what in ((o2, st2, "workspace"), (o3, st3, "allocation-free")):
        assert np.array_equal(host(o), host(o1)), f"{what}: o"
        for name in names:
            a, b = host(getattr(st, name)), host(getattr(st1, name))
            if name.startswith("buf"):  # slots past the open window's r writes are not written
                a, b = a[:, :, :r], b[:, :, :r]
            assert np.array_equal(a, b, equal_nan=True), f"{what}: {name}"
    assert np.all(host(st2.fill) == r)


def test_chunked_whole_windows_with_window_buffer():
    """T a multiple of the window and the buffer given: the state and outputs
    are bitwise those of the call without the buffer, and every fill is 0
    (an empty window buffer for decode to continue from)."""
    B, H, d, T, window = 2, 3, 128, 128, 32
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=210)
    c0, s0 = _random_state(B, H, d, 211)
    args = _inputs(x)
    o1, c1, s1 = ops.prefill_chunked(*args, window=window, chunk=32, init_codes=dev(c0), init_scales=dev(s0),
                                     out_dtype=torch.float32)
    st = _fresh(B, H, d, window)
    st.fill.fill_(7)
    o2, c2, s2 = ops.prefill_chunked(*args, window=window, chunk=32, init_codes=dev(c0), init_scales=dev(s0),
                                     out_dtype=torch.float32, state=st)
    torch.cuda.synchronize()
    assert np.array_equal(host(o1), host(o2))
    assert np.array_equal(host(c1), host(c2)) and np.array_equal(host(s1), host(s2))
    assert not host(st.fill).any()
