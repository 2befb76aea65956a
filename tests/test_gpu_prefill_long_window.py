"""GPU parity of the chunked GDN prefill with windows that are not one
64-position chunk (windows of 80, 96, 128, 256 tokens and one of a single
token: between the chunks of a window the state stays fp32; a window that is
not a multiple of 64 is padded at its end with writes that leave the state
unchanged) and with GDNQ_FLAG_NO_REQUANT (the state is never requantized and
comes back in fp32), against the CPU oracle's token-by-token recurrence,
through the C ABI.

Bars as in tests/test_gpu_prefill.py: outputs (fp32) 1e-3 per output vector
(bf16 output: 2e-2); teacher-forced requantization codes +-1 on <= 0.1% and
scales 1e-5; free-running scales within gpu_util.FREE_SCALE_DRIFT.  The fp32
state of GDNQ_FLAG_NO_REQUANT is held to the output bar, 1e-3 per state row
(max |difference| over the row / max |oracle| over the row).
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (DEV, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_free_scales, assert_scales, dev,
                      host, max_rel_err)

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops

from test_gpu_prefill_window import _inputs, _pack, _unpack


def _state(B, H, d, seed, qmax=127, rot=False):
    S = (np.random.default_rng(seed).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    S[B - 1, 0, 1] = 0.0  # a zero row
    if rot:
        S = O.gdnq_oracle.rotate(S, np.float32)
    return O.quantize_rows(S, qmax=qmax)


def _row_err(got, ref):
    """max over rows of max |got - ref| / max |ref| (rows: the last axis)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.abs(ref).max(-1)
    num = np.abs(got - ref).max(-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


@pytest.mark.parametrize("W,C,d,bits", [(128, 64, 128, 8), (256, 64, 128, 8), (128, 32, 64, 8), (128, 64, 128, 4),
                                        (80, 16, 128, 8), (96, 32, 64, 4), (1, 16, 128, 8)])
def test_long_window_teacher_forced(W, C, d, bits):
    """B=2, H=3, three windows, one window per call, each from the GPU's
    previous state (the first from a random stored state); guard zones
    around every output."""
    B, H, n = 2, 3, 3 if W > 1 else 5
    qmax = 127 if bits == 8 else 7
    x = wl.gdn_prefill(B=B, T=W * n, H=H, dk=d, dv=d, seed=80 + W + d + bits)
    codes, scales = _state(B, H, d, 81, qmax)
    cb = d * bits // 8
    for c in range(n):
        print(f"W={W} C={C} d={d} bits={bits} window {c}", flush=True)
        xs = {k: np.ascontiguousarray(v[:, c * W:(c + 1) * W]) for k, v in x.items()}
        o = Guarded((B, W, H, d), torch.float32)
        cg = Guarded((B, H, d, cb), torch.int8)
        sg = Guarded((B, H, d), torch.float32)
        ops.prefill_chunked(*_inputs(xs), window=W, chunk=C, init_codes=dev(_pack(codes, bits)),
                            init_scales=dev(scales), out_dtype=torch.float32, o=o.t, codes=cg.t, scales=sg.t,
                            state_bits=bits)
        torch.cuda.synchronize()
        assert o.guards_intact() and cg.guards_intact() and sg.guards_intact()
        ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W, codes0=codes, scale0=scales,
                        qmax=qmax)
        err = max_rel_err(host(o.t), ref["o"])
        assert err <= OUT_TOL_F32, f"window {c}: o max relative error {err:.3e}"
        assert_codes(_unpack(host(cg.t), bits), ref["codes"], f"window {c} codes")
        assert_scales(host(sg.t), ref["scale"], f"window {c} scales")
        codes, scales = _unpack(host(cg.t), bits), host(sg.t)


def test_long_window_free_running():
    """B=2, H=2, T=1024 at W=128 (eight windows of two chunks) in one call
    from a stored state, bf16 output, against the oracle run on its own."""
    B, H, d, T, W = 2, 2, 128, 1024, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=85)
    codes, scales = _state(B, H, d, 86)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), window=W, chunk=64, init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_BF16
    assert_codes(host(cg), ref["codes"], "final codes")
    assert_free_scales(host(sg), ref["scale"], f"W = {W}, {T // W} windows")


def test_window_equal_to_sequence_quantizes_once():
    """W = T: one requantization, at the end, of a state carried in fp32
    through eight chunks (B=2, H=3, T=512 from a stored state): the final
    codes and scales held to the teacher-forced bar."""
    B, H, d, T = 2, 3, 128, 512
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=87)
    codes, scales = _state(B, H, d, 88)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), window=T, chunk=64, init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=T, codes0=codes, scale0=scales)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_F32
    assert_codes(host(cg), ref["codes"], "codes")
    assert_scales(host(sg), ref["scale"], "scales")


def test_long_window_rotated_teacher_forced():
    """GDNQ_FLAG_WHT at W = 128: B=2, H=3, three windows, one per call, from
    the GPU's previous state (the first a random state in the rotated basis).
    The rotated operands the kernels used (read back from the workspace)
    match the oracle's rotation and bf16 rounding up to rounding ties on
    <= 0.1%; the recurrence on those operands is held to the teacher-forced
    bar."""
    B, H, d, W, n = 2, 3, 128, 128, 3
    x = wl.gdn_prefill(B=B, T=W * n, H=H, dk=d, dv=d, seed=89)
    codes, scales = _state(B, H, d, 90, rot=True)
    rows = B * W * H
    for c in range(n):
        xs = {k: np.ascontiguousarray(v[:, c * W:(c + 1) * W]) for k, v in x.items()}
        q_, k_, v_, a_, b_ = _inputs(xs)
        need = ops.prefill_workspace_size(q_, v_, window=W, chunk=64, wht=True, out_dtype=torch.float32)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        o, cg, sg = ops.prefill_chunked(q_, k_, v_, a_, b_, window=W, chunk=64, init_codes=dev(codes),
                                        init_scales=dev(scales), wht=True, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        # the rotated q and k are the last 2 * rows * 128 bf16 of the workspace
        rot = host(ws[need - 2 * rows * d * 2:]).view(np.uint16).reshape(2, B, W, H, d)
        qr, kr = (wl.bf16_to_f32(rot[i]) for i in range(2))
        for name, got, src in (("q", qr, xs["q"]), ("k", kr, xs["k"])):
            assert np.mean(got != O.round_bf16(O.gdnq_oracle.rotate(src, np.float32))) <= 1e-3, name
        ref = O.prefill(qr, kr, xs["v"], xs["alpha"], xs["beta"], W=W, codes0=codes, scale0=scales)
        err = max_rel_err(host(o), ref["o"])
        assert err <= OUT_TOL_F32, f"window {c}: o max relative error {err:.3e}"
        assert_codes(host(cg), ref["codes"], f"window {c} codes")
        assert_scales(host(sg), ref["scale"], f"window {c} scales")
        codes, scales = host(cg), host(sg)


@pytest.mark.parametrize("T,C,d,bits,init", [(512, 64, 128, 8, True), (512, 64, 128, 8, False), (80, 16, 64, 8, True),
                                             (256, 32, 128, 4, True), (0, 64, 128, 8, True), (48, 16, 128, 8, True)])
def test_no_requant(T, C, d, bits, init):
    """GDNQ_FLAG_NO_REQUANT: B=2, H=3 from a stored state (or zero), the final
    fp32 state and the outputs against the oracle with no quantization after
    the start (W = None); T = 0 returns the dequantized stored state."""
    B, H = 2, 3
    qmax = 127 if bits == 8 else 7
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=91 + T + d)
    codes, scales = _state(B, H, d, 92, qmax) if init else (None, None)
    o = Guarded((B, T, H, d), torch.float32)
    sf = Guarded((B, H, d, d), torch.float32)
    ops.prefill_chunked(*_inputs(x), chunk=C, init_codes=None if codes is None else dev(_pack(codes, bits)),
                        init_scales=None if scales is None else dev(scales), out_dtype=torch.float32, o=o.t,
                        state_f32=sf.t, state_bits=bits, no_requant=True)
    torch.cuda.synchronize()
    assert o.guards_intact() and sf.guards_intact()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=None, codes0=codes, scale0=scales, qmax=qmax)
    if T > 0:
        err = max_rel_err(host(o.t), ref["o"])
        assert err <= OUT_TOL_F32, f"o max relative error {err:.3e}"
    serr = _row_err(host(sf.t), ref["S"])
    print(f"T={T} d={d} bits={bits}: state max row-relative error {serr:.2e}")
    assert serr <= OUT_TOL_F32
    if T == 0:
        assert np.array_equal(host(sf.t), ref["S"])


def test_no_requant_then_quantize_equals_one_window():
    """Never requantizing and quantizing the final fp32 state with the codec
    gives the W = T call's codes (+-1 on <= 0.1%) and scales (1e-5): both
    carry the same fp32 state to the end (B=2, H=2, T=256)."""
    B, H, d, T = 2, 2, 128, 256
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=95)
    codes, scales = _state(B, H, d, 96)
    _, sf = ops.prefill_chunked(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales), out_dtype=torch.float32,
                                no_requant=True)
    _, cg, sg = ops.prefill_chunked(*_inputs(x), window=T, init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.float32)
    c2, s2 = ops.quantize_state(sf.reshape(-1, d))
    torch.cuda.synchronize()
    assert_codes(host(c2).reshape(B, H, d, d), host(cg), "codes")
    assert_scales(host(s2).reshape(B, H, d), host(sg), "scales")
