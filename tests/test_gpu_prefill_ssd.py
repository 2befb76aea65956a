"""GPU parity of the SSD (scalar-decay, no delta term) chunked prefill
against the CPU oracle, through the C ABI.

  * plain bf16 q/k (no operand quantization): outputs and the final fp32
    state within 1e-3 (max relative error per vector) with fp32 output;
  * rotated + int8 q/k operands: the operand codes come from the same codec on
    rotations computed in a different summation order, so a code may flip
    (+-1) where the rotated value sits on a rounding boundary; outputs and the
    final state are held to 2e-2 (the bf16-input bar), and the quantized
    operands themselves (read from the workspace) to the code bar: +-1 on at
    most 0.1%, scales within 1e-5.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import DEV, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales, dev, host, max_rel_err

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops


def _run(x, *, int8, wht, out_dt, workspace=None):
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    return ops.prefill_chunked(q, k, v, dev(x["alpha"]), None, ssd=True, int8_qk=int8, wht=wht,
                               out_dtype=out_dt, workspace=workspace)


def _ref(x, *, int8, wht):
    return O.prefill(x["q"], x["k"], x["v"], x["alpha"], None, W=None, kind="ssd", rot=wht,
                     qk_int8=int8)


@pytest.mark.parametrize("dv", [64, 128])
def test_ssd_plain_bf16(dv):
    x = wl.ssd_prefill(B=2, T=192, H=3, dk=128, dv=dv, seed=dv)
    o, S = _run(x, int8=False, wht=False, out_dt=torch.float32)
    torch.cuda.synchronize()
    ref = _ref(x, int8=False, wht=False)
    err_o = max_rel_err(host(o), ref["o"])
    err_s = max_rel_err(host(S), ref["S"])
    assert err_o <= OUT_TOL_F32, err_o
    assert err_s <= OUT_TOL_F32, err_s


def test_ssd_plain_matches_closed_form():
    """One head, T=128: the fp64 quadratic form of the recurrence."""
    x = wl.ssd_prefill(B=1, T=128, H=1, dk=128, dv=64, seed=4)
    o, _ = _run(x, int8=False, wht=False, out_dt=torch.float32)
    torch.cuda.synchronize()
    ref = O.ssd_closed_form(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["alpha"][0, :, 0])
    assert max_rel_err(host(o)[0, :, 0], ref) <= OUT_TOL_F32


@pytest.mark.parametrize("wht", [False, True])
@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_ssd_int8_operands(wht, out_dt):
    B, T, H, dv = 2, 128, 3, 64
    x = wl.ssd_prefill(B=B, T=T, H=H, dk=128, dv=dv, seed=7)
    q = dev(x["q"], torch.bfloat16)
    need = ops.prefill_workspace_size(q, dev(x["v"], torch.bfloat16), ssd=True, int8_qk=True, wht=wht)
    ws = Guarded((need,), torch.int8)
    o, S = _run(x, int8=True, wht=wht, out_dt=out_dt, workspace=ws.t)
    torch.cuda.synchronize()
    assert ws.guards_intact()
    ref = _ref(x, int8=True, wht=wht)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_BF16
    assert max_rel_err(host(S), ref["S"]) <= OUT_TOL_BF16
    # the quantized operands the kernel used: [q codes | k codes | q scales | k scales]
    rows = B * T * H
    w = host(ws.t)
    cq = w[:rows * 128].view(np.int8).reshape(B, T, H, 128)
    ck = w[rows * 128:2 * rows * 128].view(np.int8).reshape(B, T, H, 128)
    sq = w[2 * rows * 128:2 * rows * 128 + 4 * rows].view(np.float32).reshape(B, T, H)
    sk = w[2 * rows * 128 + 4 * rows:].view(np.float32).reshape(B, T, H)
    for name, c, s in (("q", cq, sq), ("k", ck, sk)):
        src = O.gdnq_oracle.rotate(x[name], np.float32) if wht else x[name]
        rc, rs = O.quantize_rows(src)
        assert_codes(c, rc, f"{name} operand codes")
        assert_scales(s, rs, f"{name} operand scales")


def test_ssd_outlier_channels():
    """Outlier channels (x20 on 4 channels of q and k): the rotation spreads
    them before the per-row int8 quantization."""
    x = wl.ssd_prefill(B=1, T=128, H=2, dk=128, dv=64, seed=9, outlier_channels=4)
    o, S = _run(x, int8=True, wht=True, out_dt=torch.float32)
    torch.cuda.synchronize()
    ref = _ref(x, int8=True, wht=True)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_BF16
    assert max_rel_err(host(S), ref["S"]) <= OUT_TOL_BF16


def test_ssd_empty_sequence():
    q = torch.empty((2, 0, 3, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((2, 0, 3, 64), dtype=torch.bfloat16, device=DEV)
    a = torch.empty((2, 0, 3), dtype=torch.float32, device=DEV)
    S = torch.full((2, 3, 64, 128), 7.0, device=DEV)
    ops.prefill_chunked(q, q, v, a, None, ssd=True, int8_qk=True, wht=True, state_f32=S)
    torch.cuda.synchronize()
    assert not host(S).any()


def test_ssd_batch2_seq4096_heads80_sampled():
    """The SSD workload at its full size (B=2, T=4096, H=80, d_k=128,
    d_v=64, rotated int8 q/k, bf16 output) in one call, as it is timed; three
    sampled (sequence, head) pairs recomputed by the oracle over all 4096
    tokens."""
    B, T, H, dv = 2, 4096, 80, 64
    x = wl.ssd_prefill(B=B, T=T, H=H, dk=128, dv=dv, seed=0)
    o, S = _run(x, int8=True, wht=True, out_dt=torch.bfloat16)
    torch.cuda.synchronize()
    go, gs = host(o), host(S)
    assert np.isfinite(go).all() and np.isfinite(gs).all()
    for b, h in ((0, 0), (1, 41), (1, 79)):
        xs = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in ("q", "k", "v", "alpha")}
        ref = _ref(xs, int8=True, wht=True)
        err_o = max_rel_err(go[b, :, h], ref["o"][0, :, 0])
        err_s = max_rel_err(gs[b, h], ref["S"][0, 0])
        assert err_o <= OUT_TOL_BF16, f"(b={b}, h={h}) o error {err_o:.3e}"
        assert err_s <= OUT_TOL_BF16, f"(b={b}, h={h}) state error {err_s:.3e}"
