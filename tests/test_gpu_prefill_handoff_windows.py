"""GPU parity of the prefill hand-over (gdnq_prefill_handoff) with decode's
windows below 64, at d = 64, and with the rotation, through the C ABI.

A window below 64 runs padded (every window one 64-position chunk of writes
that leave the state unchanged past its end) and the open last window of
T mod W tokens is a partial chunk whose writes go to decode's window buffer
of W slots.  Against the oracle's token-by-token recurrence with the same
window: outputs (fp32) within 1e-3 before the first window close (2e-2
after it: each side then runs from its own requantized state); codes +-1 on
<= 0.1% and scales 1e-5 when at most one window closes (one requantization
from the same stored state), else free-running scales within 2/127; fills
T mod W; buffered writes
bitwise (fp32: the bf16 inputs exactly; bf16 and FP8 buffers: the oracle's
encodings); decode then continues the sequence, each step teacher-forced.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (DEV, OUT_TOL_BF16, OUT_TOL_F32, assert_codes, assert_free_scales, assert_scales, dev, host,
                      max_rel_err)

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops

from test_gpu_prefill_handoff_bufs import _check_buffers, _dtype, _stored
from test_gpu_prefill_window import _pack, _unpack


def _inputs(x):
    return (dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
            dev(x["alpha"]), dev(x["beta"]))


def _state(B, H, d, seed, qmax=127):
    S = (np.random.default_rng(seed).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    return O.quantize_rows(S, qmax=qmax)


def _check(st, o, ref, W, T, bits, strict):
    r = T % W
    if T:
        # outputs after a window close come from each side's own requantized
        # state (codes may differ by one on a few entries): the bf16 bar there
        err = max_rel_err(host(o), ref["o"])
        assert err <= (OUT_TOL_F32 if T < W else OUT_TOL_BF16), f"o max relative error {err:.3e}"
    assert ref["n"] == r and np.all(host(st.fill) == r)
    assert_codes(_unpack(host(st.codes), bits), ref["codes"], "codes at the last boundary")
    if strict:
        assert_scales(host(st.scales), ref["scale"], "scales at the last boundary")
    else:
        assert_free_scales(host(st.scales), ref["scale"], "scales at the last boundary")
    for name, key in (("buf_k", "k"), ("buf_v", "v"), ("buf_alpha", "alpha"), ("buf_beta", "beta")):
        assert np.array_equal(host(getattr(st, name))[:, :, :r], ref["buf"][key]), name


@pytest.mark.parametrize("W,d,bits,C", [(16, 128, 8, 16), (33, 128, 8, 32), (48, 64, 8, 16), (64, 64, 8, 64),
                                        (16, 64, 4, 16), (1, 128, 8, 16)])
def test_handoff_window_matches_oracle(W, d, bits, C):
    """B=2, H=3 from a stored state; T = r, W + r and 3 W + r tokens (r =
    T mod W, the open window): outputs, the boundary state and the buffered
    writes against the oracle."""
    B, H = 2, 3
    qmax = 127 if bits == 8 else 7
    r = (5 * W) // 7
    for T in (r, W + r, 3 * W + r):
        print(f"W={W} d={d} bits={bits} C={C} T={T}", flush=True)
        x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=100 + T + W + d)
        codes, scales = _state(B, H, d, 101 + T, qmax)
        o, st = ops.prefill_handoff(*_inputs(x), window=W, chunk=C, init_codes=dev(_pack(codes, bits)),
                                    init_scales=dev(scales), out_dtype=torch.float32, state_bits=bits)
        torch.cuda.synchronize()
        ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales, qmax=qmax)
        _check(st, o, ref, W, T, bits, strict=T < 2 * W)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_handoff_window16_d64_buffer_formats(fmt):
    """d = 64, W = 16, T = 3 * 16 + 11 into bf16 / FP8 window buffers: outputs
    and boundary state equal the fp32-buffer hand-over bitwise, the buffered
    writes the oracle's encodings (FP8: a 64-element vector's scale from
    its own absmax)."""
    B, H, d, W, T = 2, 3, 64, 16, 59
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=110)
    codes, scales = _state(B, H, d, 111)
    kw = dict(window=W, chunk=16, init_codes=dev(codes), init_scales=dev(scales), out_dtype=torch.float32)
    o32, st32 = ops.prefill_handoff(*_inputs(x), **kw)
    o, st = ops.prefill_handoff(*_inputs(x), buf_dtype=_dtype(fmt), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o32) and torch.equal(st.codes, st32.codes) and torch.equal(st.scales, st32.scales)
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    assert np.all(host(st.fill) == T % W)
    _check_buffers(st, fmt, ref["buf"], T % W)


@pytest.mark.parametrize("W,d", [(16, 64), (16, 128), (40, 128)])
def test_handoff_window_then_decode(W, d):
    """Prefill T = 2 W + 5 tokens with the hand-over at window W, then 3 W
    decode steps on the GPU's state (crossing window closes), against the
    oracle's decode: each step teacher-forced (the oracle starts from the
    GPU's state before the step)."""
    B, H, steps = 2, 2, 3 * W
    T = 2 * W + 5
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=120 + W + d)
    o, st = ops.prefill_handoff(*_inputs(x), window=W, chunk=16, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.all(host(st.fill) == T % W)
    n_close = 0
    for t in range(steps):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=121 + W)
        before = [host(z).copy() for z in (st.codes, st.scales, st.buf_k, st.buf_v, st.buf_alpha,
                                           st.buf_beta, st.fill)]
        go = host(st.step(dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16),
                          dev(y["v"], torch.bfloat16), dev(y["alpha"]), dev(y["beta"]),
                          out_dtype=torch.float32))
        ro, rc, rs, *_ = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *before, W)
        assert max_rel_err(go, ro) <= OUT_TOL_BF16, f"step {t}"
        closing = before[6] + 1 == W
        if closing.any():
            n_close += 1
            assert_codes(host(st.codes)[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
    assert n_close >= 2


@pytest.mark.parametrize("W", [64, 32])
def test_handoff_rotated(W):
    """GDNQ_FLAG_WHT: B=2, H=3 from a stored state in the rotated basis, T =
    W + 21.  The rotated operands the kernels used (read back from the
    workspace) match the oracle's rotation and bf16 rounding up to rounding
    ties on <= 0.1%; on those operands the outputs, the boundary state and
    the buffered keys (the rotated keys, as decode keeps them) match the
    oracle."""
    B, H, d = 2, 3, 128
    T = W + 21
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=130 + W)
    S = (np.random.default_rng(131).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(S, np.float32))
    q_, k_, v_, a_, b_ = _inputs(x)
    p = ops._prefill_params(q_, v_, window=W, chunk=64, wht=True, ssd=False, int8_qk=False,
                            out_dtype=torch.float32)
    need = int(ops._lib.prefill_handoff_workspace_size(p))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o, st = ops.prefill_handoff(q_, k_, v_, a_, b_, window=W, init_codes=dev(codes), init_scales=dev(scales),
                                out_dtype=torch.float32, wht=True, workspace=ws)
    torch.cuda.synchronize()
    Tp = T // W * 64 + T % W  # positions of the padded run (the open window unpadded)
    rows = B * Tp * H
    rot = host(ws[need - 2 * rows * d * 2:]).view(np.uint16).reshape(2, B, Tp, H, d)
    real = np.concatenate([np.arange(w * 64, w * 64 + W) for w in range(T // W)] + [np.arange(T // W * 64, Tp)])
    qr, kr = (wl.bf16_to_f32(rot[i][:, real]) for i in range(2))
    for name, got, src in (("q", qr, x["q"]), ("k", kr, x["k"])):
        assert np.mean(got != O.round_bf16(O.gdnq_oracle.rotate(src, np.float32))) <= 1e-3, name
    ref = O.prefill(qr, kr, x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    _check(st, o, ref, W, T, 8, strict=True)
    assert st.wht


KEYS = ("q", "k", "v", "alpha", "beta")


def _check_sequence(st, b, o_new, ref, W, n_close, what):
    """Sequence b of a packed / resumed call against the oracle's run of it
    (ref: outputs of its new tokens, codes, scales, buffer)."""
    r = ref["n"]
    assert host(st.fill)[b] == r, f"{what}: fill"
    if o_new.shape[0]:
        err = max_rel_err(host(o_new), ref["o"])
        assert err <= (OUT_TOL_F32 if n_close == 0 else OUT_TOL_BF16), f"{what}: o max relative error {err:.3e}"
    assert_codes(host(st.codes)[b], ref["codes"][0], f"{what} codes")
    if n_close <= 1:
        assert_scales(host(st.scales)[b], ref["scale"][0], f"{what} scales")
    else:
        assert_free_scales(host(st.scales)[b], ref["scale"][0], f"{what} scales")
    for name, key in (("buf_k", "k"), ("buf_v", "v"), ("buf_alpha", "alpha"), ("buf_beta", "beta")):
        assert np.array_equal(host(getattr(st, name))[b, :, :r], ref["buf"][key][0]), (what, name)


@pytest.mark.parametrize("W,d", [(16, 128), (16, 64), (64, 64), (37, 128)])
def test_varlen_window(W, d):
    """Packed sequences (empty, one token, W - 1, W, 3 W + 5, 70 and 130
    tokens; H=3) from stored states at decode's window W: each padded on the
    device (whole windows to 64 positions, the open one unpadded) and every
    sequence against the oracle run on it alone."""
    H = 3
    lengths = [0, 1, W - 1, W, 3 * W + 5, 70, 130]
    B = len(lengths)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=140 + W + d)
    codes, scales = _state(B, H, d, 141)
    cu = x["cu_seqlens"]
    o, st = ops.prefill_varlen(*_inputs(x), dev(cu), window=W, init_codes=dev(codes), init_scales=dev(scales),
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        ref = O.prefill(*(x[key][None, t0:t1] for key in KEYS), W=W, codes0=codes[b:b + 1], scale0=scales[b:b + 1])
        ref["o"] = ref["o"][0]
        ref["buf"] = {k: v for k, v in ref["buf"].items()}
        _check_sequence(st, b, o[t0:t1], ref, W, (t1 - t0) // W, f"W={W} d={d} sequence {b} ({t1 - t0} tokens)")


@pytest.mark.parametrize("W,d,packed", [(16, 128, False), (16, 64, True), (32, 64, False), (64, 64, True)])
def test_resume_window(W, d, packed):
    """Decode states of window W at fills 0, W / 2 and W - 1 (buffered bf16
    writes) resume with 2 W + 7 new tokens each (packed: 0, W + 3 and 3 W
    tokens): the open window's buffered writes and the new tokens form one
    sequence whose windows start at the first buffered write, padded on the
    device; every sequence against the oracle over its buffered writes and
    new tokens from the stored state."""
    H = 2
    fills = [0, W // 2, W - 1]
    B = len(fills)
    g = np.random.default_rng(150 + W + d)
    codes, scales = O.quantize_rows((g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32))
    pre = wl.gdn_prefill(B=B, T=W, H=H, dk=d, dv=d, seed=151)
    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(np.asarray(fills, np.int32)))
    bk = np.zeros((B, H, W, d), np.float32)
    bv = np.zeros((B, H, W, d), np.float32)
    ba = np.zeros((B, H, W), np.float32)
    bb = np.zeros((B, H, W), np.float32)
    for b, f in enumerate(fills):
        bk[b, :, :f] = np.moveaxis(pre["k"][b, :f], 0, 1)
        bv[b, :, :f] = np.moveaxis(pre["v"][b, :f], 0, 1)
        ba[b, :, :f] = pre["alpha"][b, :f].T
        bb[b, :, :f] = pre["beta"][b, :f].T
    for name, val in (("buf_k", bk), ("buf_v", bv), ("buf_alpha", ba), ("buf_beta", bb)):
        getattr(st, name).copy_(dev(val))
    if packed:
        lengths = [0, W + 3, 3 * W]
        x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=152)
        cu = x["cu_seqlens"]
        o = ops.prefill_resume(st, *(dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None) for key in KEYS),
                               cu_seqlens=dev(cu), out_dtype=torch.float32)
        new = [{key: x[key][int(cu[b]):int(cu[b + 1])] for key in KEYS} for b in range(B)]
        outs = [o[int(cu[b]):int(cu[b + 1])] for b in range(B)]
    else:
        T = 2 * W + 7
        x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=152)
        o = ops.prefill_resume(st, *(dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None) for key in KEYS),
                               out_dtype=torch.float32)
        new = [{key: x[key][b] for key in KEYS} for b in range(B)]
        outs = [o[b] for b in range(B)]
    torch.cuda.synchronize()
    for b, f in enumerate(fills):
        n = new[b]["q"].shape[0]
        seq = {key: np.concatenate([pre[key][b, :f], new[b][key]])[None] for key in KEYS}
        ref = O.prefill(*(seq[key] for key in KEYS), W=W, codes0=codes[b:b + 1], scale0=scales[b:b + 1])
        ref["o"] = ref["o"][0, f:]
        _check_sequence(st, b, outs[b], ref, W, (f + n) // W, f"W={W} d={d} sequence {b} (fill {f}, {n} new)")
