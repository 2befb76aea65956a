"""GPU parity of the uniform 4-bit state (GDNQ_FLAG_STATE_4BIT: codec with
scale = absmax / 7 and codes in [-7, 7], two per byte) for the codec, the
decode step and the GDN prefill (chunked, hand-over, resume), against the
oracle's qmax = 7 option.  Codes are compared after
unpacking the nibbles here; the bars are those of the 8-bit state (codes
bitwise where the decision is exact, +-1 on <= 0.1% after a replayed close;
scales 1e-5; outputs 1e-3 / 2e-2)."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (DEV, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales,
                      dev, host, max_rel_err)

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops


def pack4(codes):
    """int8 codes in [-7, 7], [..., d] -> packed bytes [..., d/2] (column
    2j in the low nibble of byte j)."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8).view(np.int8)


def unpack4(packed):
    b = np.asarray(packed).view(np.uint8).astype(np.int16)
    lo, hi = b & 0xF, b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int16)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out.astype(np.int8)


def test_pack4_roundtrip():
    g = np.random.default_rng(1)
    c = g.integers(-7, 8, (5, 128)).astype(np.int8)
    assert np.array_equal(unpack4(pack4(c)), c)
    assert pack4(np.array([[1, -1]], np.int8)).view(np.uint8).tolist() == [[0xF1]]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [1, 17, 4099])
@pytest.mark.parametrize("wht", [False, True])
def test_codec4_random(d, rows, wht):
    g = np.random.default_rng(rows + d + 4)
    S = (g.standard_normal((rows, d)) * np.exp(g.uniform(-4, 4, (rows, 1)))).astype(np.float32)
    S[rows // 2] = 0.0
    St = Guarded((rows, d), torch.float32).set(S)
    C = Guarded((rows, d // 2), torch.int8)
    Sc = Guarded((rows,), torch.float32)
    ops.quantize_state(St.t, C.t, Sc.t, wht=wht, state_bits=4)
    torch.cuda.synchronize()
    assert C.guards_intact() and Sc.guards_intact()
    rc, rs = O.quantize_rows(O.gdnq_oracle.rotate(S, np.float32) if wht else S, qmax=7)
    got = unpack4(host(C.t))
    if wht:
        assert_codes(got, rc, "codec4+wht")
        assert_scales(host(Sc.t), rs, "codec4+wht")
    else:
        assert np.array_equal(got, rc)
        assert np.array_equal(host(Sc.t), rs)


CASES = [
    # (B, H, dk, dv, W, in_dtype, out_dtype, wht, fills)
    (4, 3, 128, 128, 8, torch.bfloat16, torch.bfloat16, False, [0, 3, 7, 7]),
    (4, 3, 128, 128, 8, torch.bfloat16, torch.float32, True, [7, 1, 6, 0]),
    (3, 2, 128, 64, 5, torch.bfloat16, torch.bfloat16, False, [4, 2, 0]),
    (3, 2, 64, 128, 5, torch.float32, torch.float32, False, [4, 2, 0]),
    (2, 5, 64, 64, 16, torch.float32, torch.float32, True, [15, 9]),
    (2, 2, 128, 128, 64, torch.bfloat16, torch.bfloat16, False, [63, 62]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}dk{c[2]}dv{c[3]}W{c[4]}wht{int(c[7])}")
def test_decode4_step_cases(case):
    """One step from a stored 4-bit state with buffered writes, some
    sequences closing their window: outputs, closed rows (requantized with
    the 4-bit codec), untouched rows bitwise, appended writes exact."""
    B, H, dk, dv, W, in_dt, out_dt, wht, fills = case
    d = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=B * 7 + W + 4, fill=np.array(fills))
    if in_dt == torch.float32:
        g = np.random.default_rng(W + 4)
        d["q"] = wl.l2norm(g.standard_normal(d["q"].shape).astype(np.float32))
        d["k"] = wl.l2norm(g.standard_normal(d["k"].shape).astype(np.float32))
        d["v"] = g.standard_normal(d["v"].shape).astype(np.float32)
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(d["state"], np.float32) if wht else d["state"],
                                    qmax=7)
    gc = Guarded((B, H, dv, dk // 2), torch.int8).set(pack4(codes))
    gs = Guarded((B, H, dv), torch.float32).set(scales)
    bk, bv = dev(d["buf_k"]), dev(d["buf_v"])
    ba, bb = dev(d["buf_alpha"]), dev(d["buf_beta"])
    fout = torch.empty(B, dtype=torch.int32, device=DEV)
    o = Guarded((B, H, dv), out_dt)
    ops.decode_step(dev(d["q"], in_dt), dev(d["k"], in_dt), dev(d["v"], in_dt), dev(d["alpha"]),
                    dev(d["beta"]), gc.t, gs.t, bk, bv, ba, bb, dev(d["fill"]), fout, o.t, wht=wht)
    torch.cuda.synchronize()
    assert gc.guards_intact() and gs.guards_intact() and o.guards_intact()
    ro, rc, rs, rbk, rbv, rba, rbb, rfill = O.decode_step(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes, scales, d["buf_k"], d["buf_v"],
        d["buf_alpha"], d["buf_beta"], d["fill"], W, rot=wht, qmax=7)
    tol = OUT_TOL_F32 if (in_dt == torch.float32 and out_dt == torch.float32) else OUT_TOL_BF16
    err = max_rel_err(host(o.t), ro)
    assert err <= tol, f"o max relative error {err:.3e}"
    assert np.array_equal(host(fout), rfill)
    got_c, got_s = unpack4(host(gc.t)), host(gs.t)
    closing = d["fill"] + 1 == W
    assert np.array_equal(got_c[~closing], codes[~closing])
    assert np.array_equal(got_s[~closing], scales[~closing])
    if closing.any():
        assert np.abs(got_c).max() <= 7
        assert_codes(got_c[closing], rc[closing], "closing 4-bit codes")
        assert_scales(got_s[closing], rs[closing], "closing scales")
    for bi in np.nonzero(~closing)[0]:
        f = d["fill"][bi]
        assert np.array_equal(host(bv)[bi, :, f], rbv[bi, :, f])
        assert np.array_equal(host(ba)[bi, :, f], rba[bi, :, f])


@pytest.mark.parametrize("buf", ["fp32", "bf16", "fp8"])
def test_decode4_windows_teacher_forced(buf):
    """B=3 H=4 d=128 W=8 for 26 steps (three closes per sequence at
    staggered fills), each step against the oracle from the GPU's state
    before it, with the fp32, bf16 and FP8 window buffers."""
    B, H, d, W, steps = 3, 4, 128, 8, 26
    g = np.random.default_rng(11)
    codes, scales = O.quantize_rows((g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32), qmax=7)
    bdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[buf]
    st = ops.DecodeState(dev(pack4(codes)), dev(scales), W, fill=dev(np.array([0, 3, 6], np.int32)),
                         buf_dtype=bdt, state_bits=4)
    for x in (st.buf_k, st.buf_v):  # the writes already buffered are identities (alpha 1, beta 0)
        x.zero_()
    st.buf_alpha.fill_(1.0)
    st.buf_beta.zero_()
    if buf == "fp8":
        st.buf_k_scale.zero_()
        st.buf_v_scale.zero_()

    def buffers():
        k, v = host(st.buf_k), host(st.buf_v)
        if buf == "fp8":
            k = k * host(st.buf_k_scale)[..., None]
            v = v * host(st.buf_v_scale)[..., None]
        return k, v

    n_close = 0
    for t in range(steps):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=12)
        bk, bv = buffers()
        before = [unpack4(host(st.codes)), host(st.scales).copy(), bk, bv, host(st.buf_alpha).copy(),
                  host(st.buf_beta).copy(), host(st.fill).copy()]
        go = host(st.step(dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16),
                          dev(y["v"], torch.bfloat16), dev(y["alpha"]), dev(y["beta"]),
                          out_dtype=torch.float32))
        ro, rc, rs, *_ = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *before, W,
                                      buf_bf16=buf == "bf16", buf_fp8=buf == "fp8", qmax=7)
        err = max_rel_err(go, ro)
        assert err <= OUT_TOL_BF16, (t, err)
        closing = before[6] + 1 == W
        if closing.any():
            n_close += 1
            assert_codes(unpack4(host(st.codes))[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
    assert n_close >= 6


def test_decode4_batch64_heads32_window64():
    """The bench shape with the 4-bit state: B=64 H=32 d=128 W=64, fills
    U{0..63} with five sequences at 63: outputs and the closing sequences
    against the oracle."""
    B, H, d, W = 64, 32, 128, 64
    fill = np.random.default_rng(3).integers(0, W, B)
    fill[[0, 9, 20, 41, 63]] = W - 1
    x = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=3, fill=fill)
    codes, scales = O.quantize_rows(x["state"], qmax=7)
    st = ops.DecodeState(dev(pack4(codes)), dev(scales), W, fill=dev(x["fill"]), state_bits=4)
    st.buf_k.copy_(dev(np.nan_to_num(x["buf_k"])))
    st.buf_v.copy_(dev(np.nan_to_num(x["buf_v"])))
    st.buf_alpha.copy_(dev(np.nan_to_num(x["buf_alpha"])))
    st.buf_beta.copy_(dev(np.nan_to_num(x["buf_beta"])))
    go = host(st.step(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16),
                      dev(x["v"], torch.bfloat16), dev(x["alpha"]), dev(x["beta"]),
                      out_dtype=torch.float32))
    ro, rc, rs, *_ = O.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], codes, scales,
                                   x["buf_k"], x["buf_v"], x["buf_alpha"], x["buf_beta"], x["fill"], W,
                                   qmax=7)
    assert max_rel_err(go, ro) <= OUT_TOL_BF16
    closing = x["fill"] + 1 == W
    assert closing.any()
    assert_codes(unpack4(host(st.codes))[closing], rc[closing], "closing codes")
    assert_scales(host(st.scales)[closing], rs[closing], "closing scales")
    assert np.array_equal(unpack4(host(st.codes))[~closing], codes[~closing])


# ---------------------------------------------------------------- GDN prefill with the 4-bit state
W64 = 64
KEYS = ("q", "k", "v", "alpha", "beta")


def _pf_inputs(x):
    return [dev(x[key], torch.bfloat16 if key in ("q", "k", "v") else None) for key in KEYS]


def test_prefill4_teacher_forced_chunks():
    """B=2, H=3, four chunks, one per call from the GPU's previous 4-bit
    state (the first from a random stored one): every window's 4-bit
    requantization against the oracle on identical inputs."""
    B, H, d, T = 2, 3, 128, 256
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=21)
    g = np.random.default_rng(22)
    codes, scales = O.quantize_rows((g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32), qmax=7)
    for c in range(T // W64):
        xs = {k: np.ascontiguousarray(v[:, c * W64:(c + 1) * W64]) for k, v in x.items()}
        cg = Guarded((B, H, d, d // 2), torch.int8)
        sg = Guarded((B, H, d), torch.float32)
        o, _, _ = ops.prefill_chunked(*_pf_inputs(xs), init_codes=dev(pack4(codes)),
                                      init_scales=dev(scales), out_dtype=torch.float32, codes=cg.t,
                                      scales=sg.t, state_bits=4)
        torch.cuda.synchronize()
        assert cg.guards_intact() and sg.guards_intact()
        ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W64, codes0=codes,
                        scale0=scales, qmax=7)
        err = max_rel_err(host(o), ref["o"])
        assert err <= OUT_TOL_F32, f"chunk {c}: o max relative error {err:.3e}"
        got = unpack4(host(cg.t))
        assert np.abs(got).max() <= 7
        assert_codes(got, ref["codes"], f"chunk {c} codes")
        assert_scales(host(sg.t), ref["scale"], f"chunk {c} scales")
        codes, scales = got, host(sg.t)


def test_prefill4_handoff_then_decode4():
    """4-bit hand-over of T = 100 tokens (one close, 36 open writes), then
    40 decode steps on the same 4-bit DecodeState across the next close,
    each teacher-forced against the oracle."""
    B, H, d, T = 2, 2, 128, 100
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=23)
    o, st = ops.prefill_handoff(*_pf_inputs(x), out_dtype=torch.float32, state_bits=4)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W64, qmax=7)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_BF16
    assert np.all(host(st.fill) == T % W64)
    assert_codes(unpack4(host(st.codes)), ref["codes"], "hand-over codes")
    assert_scales(host(st.scales), ref["scale"], "hand-over scales")
    n_close = 0
    for t in range(40):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=24)
        before = [unpack4(host(st.codes)), host(st.scales).copy(), host(st.buf_k).copy(),
                  host(st.buf_v).copy(), host(st.buf_alpha).copy(), host(st.buf_beta).copy(),
                  host(st.fill).copy()]
        go = host(st.step(dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16),
                          dev(y["v"], torch.bfloat16), dev(y["alpha"]), dev(y["beta"]),
                          out_dtype=torch.float32))
        ro, rc, rs, *_ = O.decode_step(y["q"], y["k"], y["v"], y["alpha"], y["beta"], *before, W64,
                                      qmax=7)
        assert max_rel_err(go, ro) <= OUT_TOL_BF16, t
        closing = before[6] + 1 == W64
        if closing.any():
            n_close += 1
            assert_codes(unpack4(host(st.codes))[closing], rc[closing], f"step {t} codes")
            assert_scales(host(st.scales)[closing], rs[closing], f"step {t} scales")
    assert n_close == 1


def test_prefill4_resume_split_equals_one_call():
    """With the 4-bit state too, a hand-over of 37 tokens then resuming
    with the rest equals one hand-over call bitwise."""
    B, H, d, T, T1 = 2, 2, 128, 230, 37
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=25)
    t = dict(zip(KEYS, _pf_inputs(x)))
    a_o, a_st = ops.prefill_handoff(*(t[key] for key in KEYS), out_dtype=torch.float32, state_bits=4)
    _, b_st = ops.prefill_handoff(*(t[key][:, :T1].contiguous() for key in KEYS),
                                  out_dtype=torch.float32, state_bits=4)
    b_o = ops.prefill_resume(b_st, *(t[key][:, T1:].contiguous() for key in KEYS),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a_o[:, T1:], b_o)
    for name in ("codes", "scales", "fill"):
        assert torch.equal(getattr(a_st, name), getattr(b_st, name)), name


def test_prefill4_varlen_matches_oracle():
    """A packed batch with the 4-bit state (eight sequences, B * H a
    multiple of 8, so the longest-first order runs too): every sequence's
    outputs, boundary state and open writes against the oracle."""
    H, d = 2, 128
    lengths = [5, 200, 64, 0, 130, 33, 1, 90]
    B = len(lengths)
    x = wl.gdn_prefill_varlen(lengths, H=H, dk=d, dv=d, seed=70)
    cu = x["cu_seqlens"]
    o, st = ops.prefill_varlen(*_pf_inputs(x), dev(cu), out_dtype=torch.float32, state_bits=4)
    torch.cuda.synchronize()
    codes = unpack4(host(st.codes))
    for b in range(B):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        n = t1 - t0
        ref = O.prefill(*(x[key][None, t0:t1] for key in KEYS), W=W64, qmax=7)
        assert host(st.fill)[b] == n % W64
        if n:
            err = max_rel_err(host(o)[t0:t1], ref["o"][0])
            assert err <= (OUT_TOL_F32 if n < W64 else OUT_TOL_BF16), (b, err)
        assert_codes(codes[b], ref["codes"][0], f"sequence {b} codes")
        if n < 2 * W64:
            assert_scales(host(st.scales)[b], ref["scale"][0], f"sequence {b} scales")
        r = n % W64
        assert np.array_equal(host(st.buf_k)[b, :, :r], ref["buf"]["k"][0]), b
