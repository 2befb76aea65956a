"""GPU parity of the prefill that resumes from a decode state at any fill
(gdnq_prefill_resume): a sequence whose open window already holds f buffered
writes continues with new tokens, and its first window closes after 64 - f of
them.  The oracle is the windowed recurrence over the buffered writes
followed by the new tokens, from the stored state (one run of it equals
decode calls at any point, pinned on the CPU); the outputs of the buffered
positions are decode's and are not produced here.

The buffered keys and values are bf16 values widened to fp32, as decode
stores them from bf16 inputs, so entering them at bf16 is exact.  Bars as
for the hand-over: o within 1e-3 (fp32 output) while no window closed, else
2e-2; codes +-1 on <= 0.1% and scales 1e-5 after at most one close, scales
within 2/127 after more; buffered writes and fills exact.
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
KEYS = ("q", "k", "v", "alpha", "beta")


def _decode_state(fills, H, d, seed):
    """A DecodeState of len(fills) sequences: random stored state, and the
    first fills[b] slots of each window buffer holding writes drawn like
    prefill tokens (bf16 keys and values).  Returns (state, prefix tokens)."""
    B = len(fills)
    g = np.random.default_rng(seed)
    codes, scales = O.quantize_rows((g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32))
    pre = wl.gdn_prefill(B=B, T=W, H=H, dk=d, dv=d, seed=seed + 1)  # [B, 64, H, ...]
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
    for name, x in (("buf_k", bk), ("buf_v", bv), ("buf_alpha", ba), ("buf_beta", bb)):
        getattr(st, name).copy_(dev(x))
    return st, codes, scales, pre


def _check_seq(st, o_new, pre, f, new, b, codes0, scales0):
    """Sequence b: its f buffered writes then its new tokens (dict of
    [n, H, ...] arrays), against the oracle over both from the stored
    state."""
    n = new["q"].shape[0]
    seq = {key: np.concatenate([pre[key][b, :f], new[key]])[None] for key in KEYS}
    ref = O.prefill(*(seq[key] for key in KEYS), W=W, codes0=codes0[b:b + 1],
                    scale0=scales0[b:b + 1])
    total = f + n
    r = total % W
    assert host(st.fill)[b] == r, f"sequence {b}: fill"
    if n:
        err = max_rel_err(host(o_new), ref["o"][0, f:])
        tol = OUT_TOL_F32 if total < W else OUT_TOL_BF16
        assert err <= tol, f"sequence {b} (fill {f}, {n} new): o max relative error {err:.3e}"
    codes, scales = host(st.codes)[b], host(st.scales)[b]
    assert_codes(codes, ref["codes"][0], f"sequence {b} codes")
    if total < 2 * W:
        assert_scales(scales, ref["scale"][0], f"sequence {b} scales")
    else:
        assert_free_scales(scales, ref["scale"][0], f"resume sequence {b}")
    for name, key in (("buf_k", "k"), ("buf_v", "v"), ("buf_alpha", "alpha"), ("buf_beta", "beta")):
        assert np.array_equal(host(getattr(st, name))[b, :, :r], ref["buf"][key][0]), (b, name)


@pytest.mark.parametrize("T", [0, 1, 10, 46, 47, 100, 200])
def test_resume_matches_oracle(T):
    """Three sequences at fills 0, 17 and 63 take T new tokens each (the
    63-fill one closes its window on its first new token)."""
    H, d = 2, 128
    fills = [0, 17, 63]
    B = len(fills)
    st, codes, scales, pre = _decode_state(fills, H, d, seed=T + 40)
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T + 41)
    o = ops.prefill_resume(st, *(dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None)
                                 for key in KEYS), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, f in enumerate(fills):
        _check_seq(st, o[b], pre, f, {key: x[key][b] for key in KEYS}, b, codes, scales)


@pytest.mark.parametrize("T1", [37, 64, 100])
def test_resume_split_equals_one_call(T1):
    """Hand-over of the first T1 tokens, then resuming with the rest, gives
    bitwise the second part's outputs and the final state, buffer and fill
    of one hand-over call over all tokens: the chunks fall on the same
    positions and the buffered writes are bf16 values."""
    B, H, d, T = 2, 2, 128, 230
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T1)
    t = {key: dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None) for key in KEYS}
    a_o, a_st = ops.prefill_handoff(*(t[key] for key in KEYS), out_dtype=torch.float32)
    _, b_st = ops.prefill_handoff(*(t[key][:, :T1].contiguous() for key in KEYS),
                                  out_dtype=torch.float32)
    b_o = ops.prefill_resume(b_st, *(t[key][:, T1:].contiguous() for key in KEYS),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a_o[:, T1:], b_o)
    r = T % W
    for name in ("codes", "scales", "fill"):
        assert torch.equal(getattr(a_st, name), getattr(b_st, name)), name
    for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
        assert torch.equal(getattr(a_st, name)[:, :, :r], getattr(b_st, name)[:, :, :r]), name


def test_resume_varlen():
    """Packed new tokens of different lengths at different fills, including
    a sequence with no new tokens (state, buffer and fill unchanged) and one
    that fills its window exactly."""
    H, d = 2, 128
    fills = [5, 40, 0, 63, 20]
    lengths = [100, 0, 64, 1, 44]
    B = len(fills)
    st, codes, scales, pre = _decode_state(fills, H, d, seed=77)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=78)
    cu = x["cu_seqlens"]
    o = ops.prefill_resume(st, *(dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None)
                                 for key in KEYS), cu_seqlens=dev(cu), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, f in enumerate(fills):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        _check_seq(st, o[t0:t1], pre, f, {key: x[key][t0:t1] for key in KEYS}, b, codes, scales)


def test_resume_varlen_longest_first_order():
    """Eight packed sequences at mixed fills with H = 2 (B * H a multiple of
    8: the state pass runs them longest first): each against the oracle."""
    H, d = 2, 128
    fills = [3, 0, 63, 10, 40, 0, 22, 5]
    lengths = [150, 7, 0, 64, 1, 120, 42, 90]
    B = len(fills)
    st, codes, scales, pre = _decode_state(fills, H, d, seed=90)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=91)
    cu = x["cu_seqlens"]
    o = ops.prefill_resume(st, *(dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None)
                                 for key in KEYS), cu_seqlens=dev(cu), out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, f in enumerate(fills):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        _check_seq(st, o[t0:t1], pre, f, {key: x[key][t0:t1] for key in KEYS}, b, codes, scales)


def test_resume_rotated():
    """GDNQ_FLAG_WHT: a rotated decode state (stored state in the rotated
    basis; buffered keys the rotated bf16 keys a rotated hand-over leaves) at
    fills 0, 17 and 63 resumes with 100 new tokens each.  The new tokens'
    rotated q and k (read back from the workspace) match the oracle's
    rotation up to rounding ties on <= 0.1%; on those operands, after the
    buffered writes, every sequence is held to the bars above."""
    H, d, T = 2, 128, 100
    fills = [0, 17, 63]
    B = len(fills)
    st, codes, scales, pre = _decode_state(fills, H, d, seed=450)
    g = np.random.default_rng(451)
    S = (g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(S, np.float32))
    st.codes.copy_(dev(codes))
    st.scales.copy_(dev(scales))
    st.wht = True
    # the buffered keys in the rotated basis, as bf16 values (what the rotated
    # prefill hands over)
    pre = dict(pre, k=O.round_bf16(O.gdnq_oracle.rotate(pre["k"], np.float32)))
    bk = np.zeros((B, H, W, d), np.float32)
    for b, f in enumerate(fills):
        bk[b, :, :f] = np.moveaxis(pre["k"][b, :f], 0, 1)
    st.buf_k.copy_(dev(bk))
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=452)
    t = {key: dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None) for key in KEYS}
    need = ops.prefill_resume_workspace_size(t["q"], t["v"], B, out_dtype=torch.float32, wht=True)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o = ops.prefill_resume(st, *(t[key] for key in KEYS), out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    rows = B * T * H
    rot = host(ws[need - 2 * rows * d * 2:]).view(np.uint16).reshape(2, B, T, H, d)
    qr, kr = (wl.bf16_to_f32(rot[i]) for i in range(2))
    for name, got, src in (("q", qr, x["q"]), ("k", kr, x["k"])):
        assert np.mean(got != O.round_bf16(O.gdnq_oracle.rotate(src, np.float32))) <= 1e-3, name
    xr = dict(x, q=qr, k=kr)
    for b, f in enumerate(fills):
        _check_seq(st, o[b], pre, f, {key: xr[key][b] for key in KEYS}, b, codes, scales)
