"""GPU parity of the variable-length prefill (gdnq_prefill_varlen): a packed
batch of sequences of different lengths, each handed over to decode.  The
oracle runs every sequence on its own (its windowed token-by-token
recurrence over that sequence's tokens), so a wrong token or chunk offset
anywhere in the packing shows up as a wrong sequence.

Bars as for the hand-over: o within 1e-3 (fp32 output) of the oracle, codes
+-1 on <= 0.1% and scales 1e-5 after at most one window close from a stored
state, free-running scales within 2/127 after more, buffered writes and
fills exact.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (assert_free_scales, DEV, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales, dev,
                      host, max_rel_err)

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


def _check_seq(x, cu, b, o, st, codes0=None, scale0=None):
    """Sequence b of the packed batch against the oracle run on it alone."""
    t0, t1 = int(cu[b]), int(cu[b + 1])
    n = t1 - t0
    r = n % W
    assert host(st.fill)[b] == r, f"sequence {b}: fill"
    c0 = None if codes0 is None else codes0[b:b + 1]
    s0 = None if scale0 is None else scale0[b:b + 1]
    ref = O.prefill(*(x[key][None, t0:t1] for key in ("q", "k", "v", "alpha", "beta")), W=W,
                    codes0=c0, scale0=s0)
    if n:
        err = max_rel_err(host(o)[t0:t1], ref["o"][0])
        tol = OUT_TOL_F32 if n < 64 else OUT_TOL_BF16
        assert err <= tol, f"sequence {b} (length {n}): o max relative error {err:.3e}"
    codes, scales = host(st.codes)[b], host(st.scales)[b]
    if n < 128:
        assert_codes(codes, ref["codes"][0], f"sequence {b} codes")
        assert_scales(scales, ref["scale"][0], f"sequence {b} scales")
    else:
        assert_codes(codes, ref["codes"][0], f"sequence {b} codes")
        assert_free_scales(scales, ref["scale"][0], f"varlen sequence {b}")
    for name, key in (("buf_k", "k"), ("buf_v", "v"), ("buf_alpha", "alpha"), ("buf_beta", "beta")):
        assert np.array_equal(host(getattr(st, name))[b, :, :r], ref["buf"][key][0]), (b, name)


@pytest.mark.parametrize("lengths", [
    [0, 1, 64, 100, 200, 63, 130],
    [37],
    [128, 0, 0, 65],
])
def test_varlen_matches_oracle(lengths):
    """Empty, one-token, whole-window and ragged sequences in one packed
    call from stored states: every sequence against the oracle."""
    H, d = 3, 128
    B = len(lengths)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=sum(lengths) + B)
    codes, scales = _random_state(B, H, d, B + 7)
    cu = x["cu_seqlens"]
    o, st = ops.prefill_varlen(*_inputs(x), dev(cu), init_codes=dev(codes),
                               init_scales=dev(scales), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        _check_seq(x, cu, b, o, st, codes, scales)


def test_varlen_zero_state():
    """No initial state: empty sequences keep the zero state."""
    lengths = [0, 5, 0, 70, 0]
    H, d = 2, 128
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=3)
    cu = x["cu_seqlens"]
    o, st = ops.prefill_varlen(*_inputs(x), dev(cu), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(len(lengths)):
        _check_seq(x, cu, b, o, st)


@pytest.mark.parametrize("T", [100, 192])
def test_varlen_uniform_equals_handoff(T):
    """Equal lengths packed: bitwise the outputs, state, buffer and fill of
    the uniform hand-over on the same tokens."""
    B, H, d = 3, 2, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T)
    codes, scales = _random_state(B, H, d, T + 1)
    a_o, a_st = ops.prefill_handoff(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.bfloat16)
    packed = [dev(x[key].reshape((B * T,) + x[key].shape[2:]),
                  torch.bfloat16 if key in ("q", "k", "v") else None)
              for key in ("q", "k", "v", "alpha", "beta")]
    cu = dev(np.arange(B + 1, dtype=np.int32) * T)
    b_o, b_st = ops.prefill_varlen(*packed, cu, init_codes=dev(codes), init_scales=dev(scales),
                                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a_o.reshape(B * T, H, d), b_o)
    r = T % W
    for name in ("codes", "scales", "fill"):
        assert torch.equal(getattr(a_st, name), getattr(b_st, name)), name
    for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
        assert torch.equal(getattr(a_st, name)[:, :, :r], getattr(b_st, name)[:, :, :r]), name


def test_varlen_many_sequences():
    """1500 sequences of 0 .. 100 tokens (the sequence map spans two
    1024-entry tiles): every fill and buffered write exact, and the
    sequences around the tile boundary plus a seeded sample against the
    oracle."""
    H, d, B = 2, 128, 1500
    g = np.random.default_rng(17)
    lengths = g.integers(0, 101, B)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=18)
    cu = x["cu_seqlens"]
    o, st = ops.prefill_varlen(*_inputs(x), dev(cu), out_dtype=torch.float32)
    torch.cuda.synchronize()
    fill = host(st.fill)
    assert np.array_equal(fill, (lengths % W).astype(np.int32))
    bk, ba = host(st.buf_k), host(st.buf_alpha)
    for b in range(B):  # buffered keys (bf16 exact in fp32) and decays of every sequence
        r = int(fill[b])
        t1 = int(cu[b + 1])
        assert np.array_equal(bk[b, :, :r], np.moveaxis(x["k"][t1 - r:t1], 0, 1)), b
        assert np.array_equal(ba[b, :, :r], np.moveaxis(x["alpha"][t1 - r:t1], 0, 1)), b
    sample = sorted({0, 1022, 1023, 1024, 1025, B - 1} | set(g.choice(B, 10, replace=False).tolist()))
    for b in sample:
        _check_seq(x, cu, b, o, st)


def test_varlen_malformed_offsets_are_clamped():
    """Offsets that go backwards or past the tokens are read as their running
    maximum clamped to [0, T]: the result equals the call with those
    sanitized offsets, bitwise, and nothing outside the buffers is touched."""
    H, d, T = 2, 128, 300
    x = wl.gdn_prefill(B=1, T=T, H=H, dk=d, dv=d, seed=9)
    packed = [dev(x[key][0], torch.bfloat16 if key in ("q", "k", "v") else None)
              for key in ("q", "k", "v", "alpha", "beta")]
    bad = np.array([-5, 120, 80, 200, 1000, 250], np.int32)
    good = np.maximum.accumulate(np.clip(bad, 0, T)).astype(np.int32)
    outs = []
    for cu in (bad, good):
        go = Guarded((T, H, d), torch.float32).set(np.zeros((T, H, d), np.float32))
        _, st = ops.prefill_varlen(*packed, dev(cu), o=go.t, out_dtype=torch.float32)
        outs.append((go, st))
    torch.cuda.synchronize()
    (g1, s1), (g2, s2) = outs
    assert g1.guards_intact() and g2.guards_intact()
    o1, o2 = g1.t, g2.t
    assert torch.equal(o1, o2)
    for name in ("codes", "scales", "fill", "buf_k", "buf_alpha"):
        a, b = getattr(s1, name), getattr(s2, name)
        if name.startswith("buf"):
            r = host(s2.fill)
            for i in range(len(r)):
                assert torch.equal(a[i, :, :r[i]], b[i, :, :r[i]]), name
        else:
            assert torch.equal(a, b), name


@pytest.mark.parametrize("H", [2, 4])
def test_varlen_longest_first_order(H):
    """B = 8 sequences (B * H a multiple of 8, so the state pass takes them
    longest first, interleaved over the XCD segments): every sequence
    against the oracle from a stored state, whatever its place in the order."""
    d = 128
    lengths = [5, 200, 64, 0, 130, 33, 1, 90]
    B = len(lengths)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=H + 60)
    codes, scales = _random_state(B, H, d, H + 61)
    cu = x["cu_seqlens"]
    o, st = ops.prefill_varlen(*_inputs(x), dev(cu), init_codes=dev(codes),
                               init_scales=dev(scales), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        _check_seq(x, cu, b, o, st, codes, scales)


def test_varlen_rotated():
    """GDNQ_FLAG_WHT on a packed batch (lengths 0, 37, 100, 64 and 130, H=3,
    from stored states in the rotated basis): the rotated q and k rows the
    kernels used (all T H packed rows, read back from the workspace) match the
    oracle's rotation and bf16 rounding up to rounding ties on <= 0.1%; on
    those operands every sequence is held to the bars above, its buffered
    keys being the rotated ones."""
    lengths = [0, 37, 100, 64, 130]
    H, d = 3, 128
    B = len(lengths)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=333)
    g = np.random.default_rng(334)
    S = (g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(S, np.float32))
    cu = x["cu_seqlens"]
    q_, k_, v_, a_, b_ = _inputs(x)
    need = ops.prefill_varlen_workspace_size(q_, v_, B, out_dtype=torch.float32, wht=True)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o, st = ops.prefill_varlen(q_, k_, v_, a_, b_, dev(cu), init_codes=dev(codes), init_scales=dev(scales),
                               out_dtype=torch.float32, wht=True, workspace=ws)
    torch.cuda.synchronize()
    T = int(cu[-1])
    rows = T * H
    rot = host(ws[need - 2 * rows * d * 2:]).view(np.uint16).reshape(2, T, H, d)
    qr, kr = (wl.bf16_to_f32(rot[i]) for i in range(2))
    for name, got, src in (("q", qr, x["q"]), ("k", kr, x["k"])):
        assert np.mean(got != O.round_bf16(O.gdnq_oracle.rotate(src, np.float32))) <= 1e-3, name
    xr = dict(x, q=qr, k=kr)
    for b in range(B):
        _check_seq(xr, cu, b, o, st, codes, scales)
    assert st.wht
