"""GPU parity of the decode step with the FP8 window buffer
(GDNQ_FLAG_BUF_FP8: E4M3 vector pairs with one fp32 scale per vector)
against the oracle's buf_fp8 option, through the C ABI.

Appended writes are compared as stored values (code * scale, both sides in
fp32), bitwise, except a key rotated under WHT: the kernel's butterfly and
the oracle's dense rotation may differ in the last fp32 bit, which can move
a code by one E4M3 step and the scale by one unit in the last place.
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


class GuardedFp8:
    """An FP8 window buffer (E4M3 codes [B,H,W,d], then fp32 scales [B,H,W])
    inside one guarded allocation."""

    def __init__(self, B, H, W, d):
        n = B * H * W
        self.g = Guarded((n * d + 4 * n,), torch.uint8, fill=165)
        self.codes = self.g.t[:n * d].view(torch.float8_e4m3fn).view(B, H, W, d)
        self.scales = self.g.t[n * d:].view(torch.float32).view(B, H, W)

    def set(self, x):  # x: fp32 vectors; stored as their E4M3 vector pairs
        _, c, s = O.quantize_e4m3_vector(x)
        self.codes.copy_(dev(c).to(torch.float8_e4m3fn))
        self.scales.copy_(dev(s))
        return self

    def values(self):  # what the buffer stands for: code * scale in fp32
        return (host(self.codes) * host(self.scales)[..., None]).astype(np.float32)


def _inputs(case):
    B, H, dk, dv, W, in_dt, out_dt, wht, fills = case
    d = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=B * 13 + W, fill=np.array(fills))
    if in_dt == torch.float32:
        g = np.random.default_rng(W + 2)
        d["q"] = wl.l2norm(g.standard_normal(d["q"].shape).astype(np.float32))
        d["k"] = wl.l2norm(g.standard_normal(d["k"].shape).astype(np.float32))
        d["v"] = g.standard_normal(d["v"].shape).astype(np.float32)
    with np.errstate(invalid="ignore"):  # poisoned (NaN) slots stay NaN
        d["buf_k_fp32"], d["buf_v_fp32"] = d["buf_k"], d["buf_v"]
        d["buf_k"] = O.quantize_e4m3_vector(d["buf_k"])[0]
        d["buf_v"] = O.quantize_e4m3_vector(d["buf_v"])[0]
    return d


def _run(d, W, in_dt, out_dt, wht):
    B, H, dv, dk = d["state"].shape
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(d["state"], np.float32) if wht
                                    else d["state"])
    g = {
        "codes": Guarded((B, H, dv, dk), torch.int8).set(codes),
        "scales": Guarded((B, H, dv), torch.float32).set(scales),
        "buf_alpha": Guarded((B, H, W), torch.float32).set(d["buf_alpha"]),
        "buf_beta": Guarded((B, H, W), torch.float32).set(d["buf_beta"]),
        "fill_out": Guarded((B,), torch.int32),
        "o": Guarded((B, H, dv), out_dt),
    }
    with np.errstate(invalid="ignore"):
        bk = GuardedFp8(B, H, W, dk).set(d["buf_k_fp32"])
        bv = GuardedFp8(B, H, W, dv).set(d["buf_v_fp32"])
    fin = dev(d["fill"])
    ops.decode_step(dev(d["q"], in_dt), dev(d["k"], in_dt), dev(d["v"], in_dt), dev(d["alpha"]),
                    dev(d["beta"]), g["codes"].t, g["scales"].t, bk.codes, bv.codes,
                    g["buf_alpha"].t, g["buf_beta"].t, fin, g["fill_out"].t, g["o"].t, wht=wht)
    torch.cuda.synchronize()
    for name, x in list(g.items()) + [("buf_k", bk.g), ("buf_v", bv.g)]:
        assert x.guards_intact(), f"write outside {name}"
    out = {k: host(v.t) for k, v in g.items()}
    out["buf_k"], out["buf_v"] = bk.values(), bv.values()
    out["buf_k_scale"], out["buf_v_scale"] = host(bk.scales), host(bv.scales)
    return out, codes, scales


def _e4m3_steps(got, ref, scale):
    """Largest code difference, in E4M3 grid steps of the reference code."""
    c = np.abs(ref / np.where(scale > 0, scale, 1)[..., None])
    _, ex = np.frexp(c)
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3) * np.where(scale > 0, scale, 1)[..., None]
    return float(np.max(np.abs(got.astype(np.float64) - ref) / step))


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}dk{c[2]}dv{c[3]}W{c[4]}wht{int(c[7])}")
def test_decode_fp8_buffer_cases(case):
    B, H, dk, dv, W, in_dt, out_dt, wht, fills = case
    d = _inputs(case)
    got, codes, scales = _run(d, W, in_dt, out_dt, wht)
    o, rc, rs, rbk, rbv, rba, rbb, rfill = O.decode_step(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes, scales, d["buf_k"], d["buf_v"],
        d["buf_alpha"], d["buf_beta"], d["fill"], W, rot=wht, buf_fp8=True)
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
            rks = O.quantize_e4m3_vector(rbk[bi, :, f])[2]
            np.testing.assert_allclose(got["buf_k_scale"][bi, :, f], rks, rtol=2e-7, atol=0)
            assert _e4m3_steps(got["buf_k"][bi, :, f], rbk[bi, :, f], rks) <= 1.0 + 1e-6
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


def test_decode_fp8_buffer_batch64_heads32_window64():
    """The full-size step (B=64, H=32, d=128, W=64, drawn fills) with the FP8
    window buffer."""
    fill = wl.decode_batch(B=64, H=32, dk=128, dv=128, W=64, seed=0)["fill"]
    fill[:2] = 63
    case = (64, 32, 128, 128, 64, torch.bfloat16, torch.bfloat16, False, list(fill))
    d = _inputs(case)
    got, codes, scales = _run(d, 64, torch.bfloat16, torch.bfloat16, False)
    o, rc, rs, rbk, rbv, *_ = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes,
                                            scales, d["buf_k"], d["buf_v"], d["buf_alpha"],
                                            d["buf_beta"], d["fill"], 64, buf_fp8=True)
    err = max_rel_err(got["o"], o)
    assert err <= OUT_TOL_BF16, err
    closing = d["fill"] == 63
    assert_codes(got["codes"][closing], rc[closing], "closing codes")
    assert np.array_equal(got["codes"][~closing], codes[~closing])
    for bi in np.nonzero(~closing)[0][:8]:
        f = d["fill"][bi]
        assert np.array_equal(got["buf_k"][bi, :, f], rbk[bi, :, f])
        assert np.array_equal(got["buf_v"][bi, :, f], rbv[bi, :, f])


@pytest.mark.parametrize("wht", [False, True])
def test_decode_fp8_buffer_multi_window(wht):
    """40 steps (5 windows of 8) through DecodeState with an FP8 buffer,
    teacher-forced against the oracle's FP8-buffer step at every step."""
    B, H, dk, dv, W, T = 3, 2, 128, 128, 8, 40
    d0 = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=5, fill=np.array([0, 3, 7]))
    S0 = O.gdnq_oracle.rotate(d0["state"], np.float32) if wht else d0["state"]
    codes, scales = O.quantize_rows(S0)
    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(d0["fill"]), wht=wht,
                         buf_dtype=torch.float8_e4m3fn)
    with np.errstate(invalid="ignore"):
        for dst, sdst, x in ((st.buf_k, st.buf_k_scale, d0["buf_k"]), (st.buf_v, st.buf_v_scale, d0["buf_v"])):
            _, c, s = O.quantize_e4m3_vector(x)
            dst.copy_(dev(c).to(torch.float8_e4m3fn))
            sdst.copy_(dev(s))
    st.buf_alpha.copy_(dev(d0["buf_alpha"]))
    st.buf_beta.copy_(dev(d0["buf_beta"]))
    worst = 0.0
    for t in range(T):
        x = wl.decode_tokens(B=B, H=H, dk=dk, dv=dv, step=t, seed=11)
        bk = (host(st.buf_k) * host(st.buf_k_scale)[..., None]).astype(np.float32)
        bv = (host(st.buf_v) * host(st.buf_v_scale)[..., None]).astype(np.float32)
        before = [host(st.codes).copy(), host(st.scales).copy(), bk, bv, host(st.buf_alpha).copy(),
                  host(st.buf_beta).copy(), host(st.fill).copy()]
        o = st.step(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16),
                    dev(x["v"], torch.bfloat16), dev(x["alpha"]), dev(x["beta"]),
                    out_dtype=torch.float32)
        ro, rc, rs, _, _, _, _, rfill = O.decode_step(x["q"], x["k"], x["v"], x["alpha"],
                                                      x["beta"], *before, W, rot=wht,
                                                      buf_fp8=True)
        worst = max(worst, max_rel_err(host(o), ro))
        assert np.array_equal(host(st.fill), rfill)
        closing = before[6] + 1 == W
        if closing.any():
            assert_codes(host(st.codes)[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
    assert worst <= OUT_TOL_BF16, worst
