"""GPU parity of the decode step with the bf16 window buffer
(GDNQ_FLAG_BUF_BF16) against the oracle's buf_bf16 option, through the C ABI.

The parity bar is the one in gpu_util; buffer appends are bitwise, except a
key rotated under WHT: the kernel's butterfly and the oracle's dense
rotation may differ in the last fp32 bit, which can move the stored bf16
value by one unit in the last place.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (DEV, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales,
                      dev, host, max_rel_err)
from test_gpu_decode import DECODE_CASES

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops


def _bf16_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16


def _inputs(case):
    B, H, dk, dv, W, in_dt, out_dt, wht, fills = case
    d = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=B * 11 + W, fill=np.array(fills))
    if in_dt == torch.float32:  # fp32 inputs need not be bf16-representable
        g = np.random.default_rng(W + 1)
        d["q"] = wl.l2norm(g.standard_normal(d["q"].shape).astype(np.float32))
        d["k"] = wl.l2norm(g.standard_normal(d["k"].shape).astype(np.float32))
        d["v"] = g.standard_normal(d["v"].shape).astype(np.float32)
    d["buf_k"] = O.round_bf16(d["buf_k"])  # a bf16 buffer holds bf16 values (NaN poison stays NaN)
    d["buf_v"] = O.round_bf16(d["buf_v"])
    return d


def _run(d, W, in_dt, out_dt, wht, buf_dt):
    B, H, dv, dk = d["state"].shape
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(d["state"], np.float32) if wht
                                    else d["state"])
    g = {
        "codes": Guarded((B, H, dv, dk), torch.int8).set(codes),
        "scales": Guarded((B, H, dv), torch.float32).set(scales),
        "buf_k": Guarded((B, H, W, dk), buf_dt).set(d["buf_k"]),
        "buf_v": Guarded((B, H, W, dv), buf_dt).set(d["buf_v"]),
        "buf_alpha": Guarded((B, H, W), torch.float32).set(d["buf_alpha"]),
        "buf_beta": Guarded((B, H, W), torch.float32).set(d["buf_beta"]),
        "fill_out": Guarded((B,), torch.int32),
        "o": Guarded((B, H, dv), out_dt),
    }
    fin = dev(d["fill"])
    ops.decode_step(dev(d["q"], in_dt), dev(d["k"], in_dt), dev(d["v"], in_dt), dev(d["alpha"]),
                    dev(d["beta"]), g["codes"].t, g["scales"].t, g["buf_k"].t, g["buf_v"].t,
                    g["buf_alpha"].t, g["buf_beta"].t, fin, g["fill_out"].t, g["o"].t, wht=wht)
    torch.cuda.synchronize()
    for name, x in g.items():
        assert x.guards_intact(), f"write outside {name}"
    return {k: host(v.t) for k, v in g.items()}, codes, scales


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}dk{c[2]}dv{c[3]}W{c[4]}wht{int(c[7])}")
def test_decode_bf16_buffer_cases(case):
    B, H, dk, dv, W, in_dt, out_dt, wht, fills = case
    d = _inputs(case)
    got, codes, scales = _run(d, W, in_dt, out_dt, wht, torch.bfloat16)
    o, rc, rs, rbk, rbv, rba, rbb, rfill = O.decode_step(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes, scales, d["buf_k"], d["buf_v"],
        d["buf_alpha"], d["buf_beta"], d["fill"], W, rot=wht, buf_bf16=True)
    tol = OUT_TOL_F32 if (in_dt == torch.float32 and out_dt == torch.float32) else OUT_TOL_BF16
    err = max_rel_err(got["o"], o)
    assert err <= tol, f"o max relative error {err:.3e} > {tol}"
    assert np.array_equal(got["fill_out"], rfill)
    closing = d["fill"] + 1 == W
    assert np.array_equal(got["codes"][~closing], codes[~closing])
    assert np.array_equal(got["scales"][~closing], scales[~closing])
    for bi in np.nonzero(~closing)[0]:
        f = d["fill"][bi]
        if wht:
            gk, rk = _bf16_bits(got["buf_k"][bi, :, f]), _bf16_bits(rbk[bi, :, f])
            assert np.max(np.abs(gk.astype(np.int64) - rk.astype(np.int64))) <= 1
        else:
            assert np.array_equal(got["buf_k"][bi, :, f], rbk[bi, :, f])
        assert np.array_equal(got["buf_v"][bi, :, f], rbv[bi, :, f])
        assert np.array_equal(got["buf_alpha"][bi, :, f], rba[bi, :, f])
        assert np.array_equal(got["buf_beta"][bi, :, f], rbb[bi, :, f])
        assert np.array_equal(got["buf_k"][bi, :, :f], d["buf_k"][bi, :, :f])
        assert np.array_equal(got["buf_v"][bi, :, :f], d["buf_v"][bi, :, :f])
    if closing.any():
        assert_codes(got["codes"][closing], rc[closing], "closing codes")
        assert_scales(got["scales"][closing], rs[closing], "closing scales")


@pytest.mark.parametrize("dk,dv,W,fills", [(128, 128, 64, [63, 40, 0, 17]), (64, 64, 8, [7, 1, 4]),
                                            (128, 64, 16, [15, 3]), (64, 128, 5, [2, 4, 0])])
def test_decode_bf16_buffer_lossless_on_gpu(dk, dv, W, fills):
    """bf16 inputs, no rotation, a buffer of bf16 values: the bf16-buffer
    kernel gives exactly the fp32-buffer kernel's results (the same sweep
    pairs in the same order, read from half the bytes)."""
    B = len(fills)
    case = (B, 3, dk, dv, W, torch.bfloat16, torch.float32, False, fills)
    d = _inputs(case)
    a, _, _ = _run(d, W, torch.bfloat16, torch.float32, False, torch.float32)
    b, _, _ = _run(d, W, torch.bfloat16, torch.float32, False, torch.bfloat16)
    for name in ("o", "codes", "scales", "fill_out", "buf_alpha", "buf_beta"):
        assert np.array_equal(a[name], b[name], equal_nan=True), name
    for name in ("buf_k", "buf_v"):
        assert np.array_equal(a[name], b[name], equal_nan=True), name


def test_decode_bf16_buffer_batch64_heads32_window64():
    """The full-size step (B=64, H=32, d=128, W=64, drawn fills) with the
    bf16 window buffer."""
    fill = wl.decode_batch(B=64, H=32, dk=128, dv=128, W=64, seed=0)["fill"]
    fill[:2] = 63
    case = (64, 32, 128, 128, 64, torch.bfloat16, torch.bfloat16, False, list(fill))
    d = wl.decode_batch(B=64, H=32, dk=128, dv=128, W=64, seed=0, fill=fill)
    d["buf_k"], d["buf_v"] = O.round_bf16(d["buf_k"]), O.round_bf16(d["buf_v"])
    got, codes, scales = _run(d, 64, torch.bfloat16, torch.bfloat16, False, torch.bfloat16)
    o, rc, rs, *_ = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes, scales,
                                  d["buf_k"], d["buf_v"], d["buf_alpha"], d["buf_beta"], d["fill"],
                                  64, buf_bf16=True)
    err = max_rel_err(got["o"], o)
    assert err <= OUT_TOL_BF16, err
    closing = d["fill"] == 63
    assert_codes(got["codes"][closing], rc[closing], "closing codes")
    assert np.array_equal(got["codes"][~closing], codes[~closing])


@pytest.mark.parametrize("wht", [False, True])
def test_decode_bf16_buffer_multi_window(wht):
    """40 steps (5 windows of 8) through DecodeState with a bf16 buffer,
    teacher-forced against the oracle's bf16-buffer step at every step."""
    B, H, dk, dv, W, T = 3, 2, 128, 128, 8, 40
    d0 = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=5, fill=np.array([0, 3, 7]))
    S0 = O.gdnq_oracle.rotate(d0["state"], np.float32) if wht else d0["state"]
    codes, scales = O.quantize_rows(S0)
    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(d0["fill"]), wht=wht,
                         buf_dtype=torch.bfloat16)
    st.buf_k.copy_(dev(O.round_bf16(d0["buf_k"]), torch.bfloat16))
    st.buf_v.copy_(dev(O.round_bf16(d0["buf_v"]), torch.bfloat16))
    st.buf_alpha.copy_(dev(d0["buf_alpha"]))
    st.buf_beta.copy_(dev(d0["buf_beta"]))
    worst = 0.0
    for t in range(T):
        x = wl.decode_tokens(B=B, H=H, dk=dk, dv=dv, step=t, seed=11)
        before = [host(z).copy() for z in (st.codes, st.scales, st.buf_k, st.buf_v, st.buf_alpha,
                                           st.buf_beta, st.fill)]
        o = st.step(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16),
                    dev(x["v"], torch.bfloat16), dev(x["alpha"]), dev(x["beta"]),
                    out_dtype=torch.float32)
        ro, rc, rs, _, _, _, _, rfill = O.decode_step(x["q"], x["k"], x["v"], x["alpha"],
                                                      x["beta"], *before, W, rot=wht,
                                                      buf_bf16=True)
        worst = max(worst, max_rel_err(host(o), ro))
        assert np.array_equal(host(st.fill), rfill)
        closing = before[6] + 1 == W
        if closing.any():
            assert_codes(host(st.codes)[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
    assert worst <= OUT_TOL_BF16, worst
