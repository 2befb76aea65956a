"""The prefill hand-over, varlen and resume calls with decode's bf16 and FP8
window buffers (GDNQ_FLAG_BUF_BF16 / GDNQ_FLAG_BUF_FP8), through the C ABI.

The prefill itself does not depend on the buffer format, so its outputs and
boundary state equal the fp32-buffer call's bit for bit; the buffered writes
are held to the oracle's encodings bitwise (bf16: the inputs themselves; FP8:
quantize_e4m3_vector's codes and scales).  Decode continuing from the handed
over state is held to the oracle's decode with the same buffer option; a
resumed prefix enters the prefill at bf16 (the stored value, code * scale for
FP8, rounded to nearest even), the oracle's input likewise.
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

W = 64
KEYS = ("q", "k", "v", "alpha", "beta")
FMTS = ("bf16", "fp8")


def _dtype(fmt):
    return torch.bfloat16 if fmt == "bf16" else torch.float8_e4m3fn


def _inputs(x):
    return (dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
            dev(x["alpha"]), dev(x["beta"]))


def _stored(fmt, x):
    """What a buffer of this format holds for the writes x [..., d]:
    (values as fp32, codes, scales) -- codes/scales None for bf16."""
    if fmt == "bf16":
        return O.round_bf16(x), None, None
    vals, codes, scales = O.quantize_e4m3_vector(x)
    return vals, codes, scales


def _check_buffers(st, fmt, ref_buf, r):
    for name, key in (("buf_k", "k"), ("buf_v", "v")):
        got = getattr(st, name)[:, :, :r]
        vals, codes, scales = _stored(fmt, ref_buf[key])
        if fmt == "bf16":
            assert np.array_equal(host(got.float()), vals), name
        else:
            assert np.array_equal(host(got.view(torch.uint8)), host(dev(codes).to(torch.float8_e4m3fn).view(torch.uint8))), name
            assert np.array_equal(host(getattr(st, name + "_scale")[:, :, :r]), scales), name + " scales"
    assert np.array_equal(host(st.buf_alpha)[:, :, :r], ref_buf["alpha"])
    assert np.array_equal(host(st.buf_beta)[:, :, :r], ref_buf["beta"])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [1, 37, 100, 191])
def test_handoff_buffer_formats(fmt, T):
    """B=2, H=3 from a stored state: outputs and boundary state equal the
    fp32-buffer hand-over bitwise, fills T mod 64, buffered writes the
    oracle's encoding of its buffered writes."""
    B, H, d = 2, 3, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T + 90)
    g = np.random.default_rng(T + 91)
    codes, scales = O.quantize_rows((g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32))
    o32, st32 = ops.prefill_handoff(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.float32)
    o, st = ops.prefill_handoff(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales),
                                out_dtype=torch.float32, buf_dtype=_dtype(fmt))
    torch.cuda.synchronize()
    assert torch.equal(o, o32) and torch.equal(st.codes, st32.codes) and torch.equal(st.scales, st32.scales)
    r = T % W
    assert np.all(host(st.fill) == r)
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    assert ref["n"] == r
    _check_buffers(st, fmt, ref["buf"], r)


@pytest.mark.parametrize("fmt", FMTS)
def test_handoff_then_decode_with_buffer_format(fmt):
    """Prefill 37 tokens into a bf16/FP8 buffer, then 60 decode steps on the
    same state (one window close), against the oracle's decode with the same
    buffer option from the oracle's own prefill state: each step
    teacher-forced, the outputs also free-running."""
    B, H, d, T, steps = 2, 2, 128, 37, 60
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=93)
    o, st = ops.prefill_handoff(*_inputs(x), out_dtype=torch.float32, buf_dtype=_dtype(fmt))
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W)
    n = ref["n"]
    opt = {"buf_bf16": fmt == "bf16", "buf_fp8": fmt == "fp8"}
    bk = np.zeros((B, H, W, d), np.float32)
    bv = np.zeros((B, H, W, d), np.float32)
    ba = np.zeros((B, H, W), np.float32)
    bb = np.zeros((B, H, W), np.float32)
    bk[:, :, :n] = _stored(fmt, ref["buf"]["k"])[0]
    bv[:, :, :n] = _stored(fmt, ref["buf"]["v"])[0]
    ba[:, :, :n], bb[:, :, :n] = ref["buf"]["alpha"], ref["buf"]["beta"]
    fr = [ref["codes"], ref["scale"], bk, bv, ba, bb, np.full(B, n, np.int32)]

    def host_buf(name):
        t = getattr(st, name)
        if fmt == "fp8":
            return (host(t.float()) * host(getattr(st, name + "_scale"))[..., None]).astype(np.float32)
        return host(t.float())

    worst_tf = worst_fr = 0.0
    n_close = 0
    for t in range(steps):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=94)
        before = [host(st.codes).copy(), host(st.scales).copy(), host_buf("buf_k"), host_buf("buf_v"),
                  host(st.buf_alpha).copy(), host(st.buf_beta).copy(), host(st.fill).copy()]
        go = host(st.step(dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16), dev(y["v"], torch.bfloat16),
                          dev(y["alpha"]), dev(y["beta"]), out_dtype=torch.float32))
        ro, rc, rs, *_ = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *before, W, **opt)
        worst_tf = max(worst_tf, max_rel_err(go, ro))
        closing = before[6] + 1 == W
        if closing.any():
            n_close += 1
            assert_codes(host(st.codes)[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
        fo, *fr = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *fr, W, **opt)
        worst_fr = max(worst_fr, max_rel_err(go, fo))
    assert n_close >= 1
    assert worst_tf <= OUT_TOL_F32, worst_tf
    assert worst_fr <= OUT_TOL_BF16, worst_fr


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [10, 100])
def test_resume_from_buffer_format(fmt, T):
    """Three sequences at fills 0, 17 and 63 of a bf16/FP8 buffer take T new
    tokens each: the oracle runs the stored prefix (entered at bf16) then the
    new tokens from the stored state; new buffered writes are the format's
    encoding of the oracle's."""
    H, d = 2, 128
    fills = [0, 17, 63]
    B = len(fills)
    g = np.random.default_rng(T + 95)
    codes, scales = O.quantize_rows((g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32))
    pre = wl.gdn_prefill(B=B, T=W, H=H, dk=d, dv=d, seed=T + 96)
    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(np.asarray(fills, np.int32)), buf_dtype=_dtype(fmt))
    prefix = {key: np.zeros((B, W, H) + ((d,) if key in ("k", "v") else ()), np.float32) for key in KEYS}
    for key in ("k", "v"):
        vals, c, s = _stored(fmt, np.moveaxis(pre[key], 1, 2))  # [B, H, W, d]
        buf = getattr(st, "buf_" + key)
        if fmt == "bf16":
            buf.copy_(dev(vals, torch.bfloat16))
        else:
            buf.copy_(dev(c).to(torch.float8_e4m3fn))
            getattr(st, "buf_" + key + "_scale").copy_(dev(s))
        prefix[key] = np.moveaxis(O.round_bf16(vals), 1, 2)  # entering the prefill at bf16
    st.buf_alpha.copy_(dev(np.ascontiguousarray(np.moveaxis(pre["alpha"], 1, 2))))
    st.buf_beta.copy_(dev(np.ascontiguousarray(np.moveaxis(pre["beta"], 1, 2))))
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=T + 97)
    o = ops.prefill_resume(st, *(dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None) for key in KEYS),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, f in enumerate(fills):
        seq = {key: np.concatenate([(prefix[key] if key in ("k", "v") else pre[key])[b, :f], x[key][b]])[None]
               for key in KEYS}
        seq["q"] = np.concatenate([pre["q"][b, :f], x["q"][b]])[None]
        ref = O.prefill(*(seq[key] for key in KEYS), W=W, codes0=codes[b:b + 1], scale0=scales[b:b + 1])
        total = f + T
        r = total % W
        assert host(st.fill)[b] == r
        err = max_rel_err(host(o[b]), ref["o"][0, f:])
        assert err <= (OUT_TOL_F32 if total < W else OUT_TOL_BF16), f"sequence {b}: o {err:.3e}"
        assert_codes(host(st.codes)[b], ref["codes"][0], f"sequence {b} codes")
        if total < 2 * W:
            assert_scales(host(st.scales)[b], ref["scale"][0], f"sequence {b} scales")
        else:
            assert_free_scales(host(st.scales)[b], ref["scale"][0], f"sequence {b} scales")
        # slots below the fill that came from the prefix keep the stored bytes; new ones are encoded
        new_from = max(f - (total - r), 0)
        for name, key in (("buf_k", "k"), ("buf_v", "v")):
            got = getattr(st, name)[b, :, new_from:r]
            vals, c, s = _stored(fmt, ref["buf"][key][0][:, new_from:r])
            if fmt == "bf16":
                assert np.array_equal(host(got.float()), vals), (b, name)
            else:
                assert np.array_equal(host(got.view(torch.uint8)),
                                      host(dev(c).to(torch.float8_e4m3fn).view(torch.uint8))), (b, name)
                assert np.array_equal(host(getattr(st, name + "_scale")[b, :, new_from:r]), s), (b, name)


@pytest.mark.parametrize("fmt", FMTS)
def test_varlen_buffer_formats(fmt):
    """Eight packed sequences of seeded lengths: outputs and state equal the
    fp32-buffer call bitwise; each sequence's buffered writes are the
    format's encoding of the fp32 call's."""
    H, d = 2, 128
    lengths = np.random.default_rng(98).integers(1, 300, 8)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=99)
    args = (dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
            dev(x["alpha"]), dev(x["beta"]), dev(x["cu_seqlens"]))
    o32, st32 = ops.prefill_varlen(*args, out_dtype=torch.float32)
    o, st = ops.prefill_varlen(*args, out_dtype=torch.float32, buf_dtype=_dtype(fmt))
    torch.cuda.synchronize()
    assert torch.equal(o, o32) and torch.equal(st.codes, st32.codes) and torch.equal(st.scales, st32.scales)
    assert torch.equal(st.fill, st32.fill)
    fills = host(st.fill)
    for b, r in enumerate(fills):
        ref_buf = {key: host(getattr(st32, "buf_" + key))[b:b + 1, :, :r] for key in ("k", "v", "alpha", "beta")}
        sub = type("S", (), {})()
        for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
            setattr(sub, name, getattr(st, name)[b:b + 1])
        if fmt == "fp8":
            sub.buf_k_scale, sub.buf_v_scale = st.buf_k_scale[b:b + 1], st.buf_v_scale[b:b + 1]
        _check_buffers(sub, fmt, ref_buf, r)
