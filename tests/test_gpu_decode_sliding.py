"""GPU parity of the Pure-Write sliding window decode (GDNQ_FLAG_SLIDING;
"Low-Bit GDN Recurrent-State Quantization ...", abstract) against the CPU
oracle's decode_step_sliding, through the C ABI.

Bars: outputs within 2e-2 (bf16 inputs) or 1e-3 (fp32 inputs); every
sequence's historical state is requantized at every token, so all codes
are held to +-1 on <= 0.1% and scales to 1e-5 (teacher-forced: the oracle
starts from the GPU's state before each token); the ring slot the token
writes, bitwise; fill_out, bitwise."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import (DEV, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales, dev, host,
                      max_rel_err)

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops


def _batch(B, H, dk, dv, W, fill, seed):
    """Decode inputs with a ring buffer: slots that hold no write are NaN
    (poison: the kernel must never read them)."""
    d = wl.decode_batch(B=B, H=H, dk=dk, dv=dv, W=W, seed=seed, fill=np.minimum(fill, W - 1), poison=False)
    d["fill"] = np.asarray(fill, np.int32)
    for b in range(B):
        live = O.sliding_ring_slots(d["fill"][b], W)[0]
        dead = [s for s in range(W) if s not in live]
        for key in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
            d[key][b, :, dead] = np.nan
    return d


def _step_gpu(d, W, codes, scales, in_dt, out_dt, wht):
    B, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    g = {"codes": Guarded((B, H, dv, dk), torch.int8).set(codes),
         "scales": Guarded((B, H, dv), torch.float32).set(scales),
         "buf_k": Guarded((B, H, W, dk), torch.float32).set(d["buf_k"]),
         "buf_v": Guarded((B, H, W, dv), torch.float32).set(d["buf_v"]),
         "buf_alpha": Guarded((B, H, W), torch.float32).set(d["buf_alpha"]),
         "buf_beta": Guarded((B, H, W), torch.float32).set(d["buf_beta"]),
         "fill_out": Guarded((B,), torch.int32, fill=-1),
         "o": Guarded((B, H, dv), out_dt)}
    ops.decode_step(dev(d["q"], in_dt), dev(d["k"], in_dt), dev(d["v"], in_dt), dev(d["alpha"]), dev(d["beta"]),
                    g["codes"].t, g["scales"].t, g["buf_k"].t, g["buf_v"].t, g["buf_alpha"].t, g["buf_beta"].t,
                    dev(d["fill"]), g["fill_out"].t, g["o"].t, wht=wht, sliding=True)
    torch.cuda.synchronize()
    for name, t in g.items():
        assert t.guards_intact(), f"{name}: write outside its buffer"
    return {n: host(t.t) for n, t in g.items()}


def _check(d, W, got, codes, scales, tol, wht):
    q, k = d["q"], d["k"]
    if wht:  # the state and the buffered keys live in the rotated basis
        q, k = O.gdnq_oracle.rotate(q, np.float32), O.gdnq_oracle.rotate(k, np.float32)
    o, rc, rs, rbk, rbv, rba, rbb, rfill = O.decode_step_sliding(q, k, d["v"], d["alpha"], d["beta"], codes, scales,
                                                                 d["buf_k"], d["buf_v"], d["buf_alpha"],
                                                                 d["buf_beta"], d["fill"], W)
    err = max_rel_err(got["o"], o)
    assert err <= tol, f"o max relative error {err:.3e}"
    assert np.array_equal(got["fill_out"], rfill)
    assert_codes(got["codes"], rc, "historical codes")
    assert_scales(got["scales"], rs, "historical scales")
    for b in range(len(d["fill"])):  # the slot the token wrote
        s = O.sliding_ring_slots(d["fill"][b], W)[1]
        assert np.array_equal(got["buf_v"][b, :, s], rbv[b, :, s])
        assert np.array_equal(got["buf_alpha"][b, :, s], rba[b, :, s])
        assert np.array_equal(got["buf_beta"][b, :, s], rbb[b, :, s])
        kt = got["buf_k"][b, :, s]
        if wht:
            assert np.max(np.abs(kt - rbk[b, :, s])) <= 1e-6
        else:
            assert np.array_equal(kt, rbk[b, :, s])
    return err


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("W", [1, 5, 8, 64])
def test_sliding_step(dk, dv, W):
    """One token for sequences at every kind of fill: an empty window, a
    partly filled one, the token that fills it, full windows with the ring's
    oldest write at its start, middle and end."""
    fill = np.array(sorted({0, min(1, W - 1), W - 1, W, W + (W - 1) // 2, 2 * W - 1}), np.int32)
    d = _batch(len(fill), 3, dk, dv, W, fill, seed=dk + dv + W)
    codes, scales = O.quantize_rows(d["state"])
    got = _step_gpu(d, W, codes, scales, torch.bfloat16, torch.float32, False)
    _check(d, W, got, codes, scales, OUT_TOL_BF16, False)


@pytest.mark.parametrize("wht", [False, True])
@pytest.mark.parametrize("in_dt,out_dt,tol", [(torch.float32, torch.float32, OUT_TOL_F32),
                                              (torch.bfloat16, torch.bfloat16, OUT_TOL_BF16)])
def test_sliding_step_dtypes_rotation(wht, in_dt, out_dt, tol):
    W = 8
    fill = np.array([0, 3, 8, 11, 15], np.int32)
    d = _batch(5, 2, 128, 128, W, fill, seed=7 + int(wht))
    S0 = O.gdnq_oracle.rotate(d["state"], np.float32) if wht else d["state"]
    codes, scales = O.quantize_rows(S0)
    got = _step_gpu(d, W, codes, scales, in_dt, out_dt, wht)
    _check(d, W, got, codes, scales, tol, wht)


@pytest.mark.parametrize("W", [1, 8])
def test_sliding_consecutive_tokens(W):
    """40 consecutive tokens of 3 sequences x 2 heads, from fills 0, W-1 and
    2W-1, the ring wrapping several times.  Teacher-forced at every token
    (the oracle from the GPU's state: codes, scales, ring, fill), and a
    free-running oracle alongside for the outputs (within 2e-2)."""
    B, H, d_, T = 3, 2, 128, 40
    d0 = _batch(B, H, d_, d_, W, np.array([0, W - 1, 2 * W - 1]), seed=30 + W)
    codes, scales = O.quantize_rows(d0["state"])
    st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(d0["fill"]), sliding=True)
    for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
        getattr(st, name).copy_(dev(d0[name]))
    fr = [codes, scales, d0["buf_k"], d0["buf_v"], d0["buf_alpha"], d0["buf_beta"], d0["fill"]]
    worst_tf = worst_fr = 0.0
    for t in range(T):
        x = wl.decode_tokens(B=B, H=H, dk=d_, dv=d_, step=t, seed=33)
        before = [host(z).copy() for z in (st.codes, st.scales, st.buf_k, st.buf_v, st.buf_alpha, st.buf_beta,
                                           st.fill)]
        o = st.step(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
                    dev(x["alpha"]), dev(x["beta"]), out_dtype=torch.float32)
        go = host(o)
        ro, rc, rs, rbk, rbv, rba, rbb, rfill = O.decode_step_sliding(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                                                      *before, W)
        worst_tf = max(worst_tf, max_rel_err(go, ro))
        assert np.array_equal(host(st.fill), rfill), t
        assert_codes(host(st.codes), rc, f"token {t} codes")
        assert_scales(host(st.scales), rs, f"token {t} scales")
        fo, *fr = O.decode_step_sliding(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *fr, W)
        worst_fr = max(worst_fr, max_rel_err(go, fo))
    assert worst_tf <= OUT_TOL_BF16, worst_tf
    assert worst_fr <= OUT_TOL_BF16, worst_fr
    print(f"sliding W={W}: 40 tokens, teacher-forced {worst_tf:.2e}, free-running {worst_fr:.2e}")


def test_sliding_batch64_heads32():
    """The decode batch at its full size, B=64, H=32, d=128, with the
    sliding window of 8 writes and fills drawn U{0..15} (half the sequences
    with a full window): one token against the oracle."""
    W = 8
    fill = np.random.default_rng(50).integers(0, 2 * W, 64).astype(np.int32)
    d = _batch(64, 32, 128, 128, W, fill, seed=51)
    codes, scales = O.quantize_rows(d["state"])
    got = _step_gpu(d, W, codes, scales, torch.bfloat16, torch.bfloat16, False)
    _check(d, W, got, codes, scales, OUT_TOL_BF16, False)
