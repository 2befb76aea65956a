"""GPU parity of the chunkwise GDN prefill against the CPU oracle's token-by-
token recurrence (per-window requantization, W = chunk = 64), through the C
ABI (ops -> ctypes -> libgdnq.so).

Bars (the ones the decode tests use):
  * o: max relative error per output vector <= 1e-3 with fp32 output (bf16
    inputs are exact in both), <= 2e-2 with bf16 output;
  * teacher-forced requantization (the oracle starts from the GPU's state):
    codes +-1 on <= 0.1%, scales 1e-5;
  * free-running over several windows: codes +-1 on <= 0.1%, scales within
    2/127 (a +-1 code flip moves the next window's row absmax by at most one
    old code unit, and the transitions are non-expansive).
"""

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

W = 64


def _inputs(x):
    return (dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
            dev(x["alpha"]), dev(x["beta"]))


def _random_state(B, H, d, seed):
    g = np.random.default_rng(seed)
    S = (g.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    S[0, 0, 3] = 0.0  # one zero row
    return O.quantize_rows(S)


def _free_scale_rel(got, ref):
    return float(np.max(np.abs(got - ref) / np.where(ref > 0, ref, 1)))


@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_prefill_teacher_forced_chunks(out_dt):
    """B=2, H=3, four chunks, one chunk per call, each call from the GPU's
    previous state (the first from a random stored state): every window's
    requantization is compared on identical inputs."""
    B, H, d, T = 2, 3, 128, 256
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=1)
    codes, scales = _random_state(B, H, d, 2)
    tol = OUT_TOL_F32 if out_dt == torch.float32 else OUT_TOL_BF16
    for c in range(T // W):
        xs = {k: np.ascontiguousarray(v[:, c * W:(c + 1) * W]) for k, v in x.items()}
        o = Guarded((B, W, H, d), out_dt)
        cg = Guarded((B, H, d, d), torch.int8)
        sg = Guarded((B, H, d), torch.float32)
        ops.prefill_chunked(*_inputs(xs), init_codes=dev(codes), init_scales=dev(scales),
                            out_dtype=out_dt, o=o.t, codes=cg.t, scales=sg.t)
        torch.cuda.synchronize()
        assert o.guards_intact() and cg.guards_intact() and sg.guards_intact()
        ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W, codes0=codes,
                        scale0=scales)
        err = max_rel_err(host(o.t), ref["o"])
        assert err <= tol, f"chunk {c}: o max relative error {err:.3e}"
        assert_codes(host(cg.t), ref["codes"], f"chunk {c} codes")
        assert_scales(host(sg.t), ref["scale"], f"chunk {c} scales")
        codes, scales = host(cg.t), host(sg.t)


@pytest.mark.parametrize("init", [False, True])
def test_prefill_free_running(init):
    """B=3, H=2, T=320 (five windows) in one call, from a zero or a stored
    state, compared with the oracle run on its own."""
    B, H, d, T = 3, 2, 128, 320
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=3)
    codes = scales = None
    if init:
        codes, scales = _random_state(B, H, d, 4)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), init_codes=None if codes is None else dev(codes),
                                    init_scales=None if scales is None else dev(scales),
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    err = max_rel_err(host(o), ref["o"])
    assert err <= OUT_TOL_BF16, err
    assert_codes(host(cg), ref["codes"], "final codes")
    assert _free_scale_rel(host(sg), ref["scale"]) <= 2.0 / 127.0


def test_prefill_matches_fp64_chunk_form():
    """Single head from zero state, T=192: the fp64 chunk (UT) form of the
    oracle, requantizing per window, gives the same outputs."""
    x = wl.gdn_prefill(B=1, T=192, H=1, dk=128, dv=128, seed=9)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.chunked_fp64(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["alpha"][0, :, 0],
                         x["beta"][0, :, 0], C=64, W=64)
    err = max_rel_err(host(o)[0, :, 0], ref["o"])
    assert err <= OUT_TOL_BF16, err
    assert_codes(host(cg)[0, 0], ref["codes"], "codes vs fp64 chunk form")


def test_prefill_empty_sequence_copies_state():
    """T = 0: no output; the final state is the initial one (bitwise), or zero
    without one."""
    B, H, d = 2, 3, 128
    q = torch.empty((B, 0, H, d), dtype=torch.bfloat16, device=DEV)
    a = torch.empty((B, 0, H), dtype=torch.float32, device=DEV)
    codes, scales = _random_state(B, H, d, 6)
    o, cg, sg = ops.prefill_chunked(q, q, q, a, a, init_codes=dev(codes), init_scales=dev(scales))
    torch.cuda.synchronize()
    assert np.array_equal(host(cg), codes) and np.array_equal(host(sg), scales)
    cz = torch.full((B, H, d, d), 5, dtype=torch.int8, device=DEV)
    sz = torch.full((B, H, d), 5.0, dtype=torch.float32, device=DEV)
    ops.prefill_chunked(q, q, q, a, a, codes=cz, scales=sz)
    torch.cuda.synchronize()
    assert not host(cz).any() and not host(sz).any()


def test_prefill_in_place_continuation():
    """init_codes/init_scales may be the output buffers: two calls in place
    equal one call over both halves."""
    B, H, d, T = 2, 2, 128, 256
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=7)
    codes, scales = _random_state(B, H, d, 8)
    c_io, s_io = dev(codes), dev(scales)
    halves = []
    for lo, hi in ((0, 128), (128, 256)):
        xs = {k: np.ascontiguousarray(v[:, lo:hi]) for k, v in x.items()}
        o, _, _ = ops.prefill_chunked(*_inputs(xs), init_codes=c_io, init_scales=s_io,
                                      codes=c_io, scales=s_io, out_dtype=torch.float32)
        halves.append(host(o))
    o_all, c_all, s_all = ops.prefill_chunked(*_inputs(x), init_codes=dev(codes),
                                              init_scales=dev(scales), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate(halves, axis=1), host(o_all))
    assert np.array_equal(host(c_io), host(c_all)) and np.array_equal(host(s_io), host(s_all))


def test_prefill_state_rows_independent_of_batch():
    """Each (sequence, head) is computed alone: a sequence's outputs and state
    do not depend on the other sequences of the batch (bitwise)."""
    B, H, d, T = 3, 2, 128, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=12)
    o, c, s = ops.prefill_chunked(*_inputs(x), out_dtype=torch.float32)
    x1 = {k: np.ascontiguousarray(v[1:2]) for k, v in x.items()}
    o1, c1, s1 = ops.prefill_chunked(*_inputs(x1), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(o)[1:2], host(o1))
    assert np.array_equal(host(c)[1:2], host(c1)) and np.array_equal(host(s)[1:2], host(s1))


def test_prefill_batch4_seq8192_heads16_sampled():
    """The prefill workload at its full size (B=4, T=8192, H=16, d=128,
    chunk = window = 64, bf16 output) in one call, as it is timed.  Three
    sampled (sequence, head) pairs are recomputed by the oracle over all
    8192 tokens (free-running, 128 windows): outputs within 2e-2, final codes
    +-1 on <= 0.1%, scales within 2/127.  Every output is finite."""
    B, T, H, d = 4, 8192, 16, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=0)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    go, gc, gs = host(o), host(cg), host(sg)
    assert np.isfinite(go).all()
    for b, h in ((0, 0), (2, 7), (3, 15)):
        xs = {k: np.ascontiguousarray(v[b:b + 1, :, h:h + 1]) for k, v in x.items()}
        ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W)
        err = max_rel_err(go[b, :, h], ref["o"][0, :, 0])
        assert err <= OUT_TOL_BF16, f"(b={b}, h={h}) o error {err:.3e}"
        assert_codes(gc[b, h], ref["codes"][0, 0], f"(b={b}, h={h}) codes")
        assert _free_scale_rel(gs[b, h], ref["scale"][0, 0]) <= 2.0 / 127.0
