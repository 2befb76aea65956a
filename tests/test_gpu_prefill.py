"""GPU parity of the chunkwise GDN prefill against the CPU oracle's token-by-
token recurrence (per-window requantization, W = chunk = 64), through the C
ABI (ops -> ctypes -> libgdnq.so).

Bars (the ones the decode tests use):
  * o: max relative error per output vector <= 1e-3 with fp32 output (bf16
    inputs are exact in both), <= 2e-2 with bf16 output;
  * teacher-forced requantization (the oracle starts from the GPU's state):
    codes +-1 on <= 0.1%, scales 1e-5;
  * free-running over several windows (a diagnostic): codes +-1 on <= 0.1%,
    scales within the drift bound of gpu_util.FREE_SCALE_DRIFT.
"""

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pool
import workloads as wl
from gpu_util import (DEV, assert_free_scales, OUT_TOL_BF16, OUT_TOL_F32, Guarded, assert_codes, assert_scales,
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


def test_prefill_requantizes_subnormal_scale_rows():
    """A stored state whose row 5 has a subnormal scale (the golden row of
    tests/golden/codec_subnormal.txt) carried through one window with
    alpha = 1, beta = 0 (the state does not change): the window-end
    requantization must give back the same codes and scales, for the tiny
    row and for the ordinary rows, as the oracle does."""
    from conftest import read_golden
    g = read_golden("codec_subnormal.txt")
    f = 2.0 ** int(g["pow2"][0])
    B, H, d, T = 1, 2, 128, 64
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=31)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    S = (np.random.default_rng(32).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    vals = np.array([float(v) for v in g["row"][0].split()]) * f
    S[0, 1, 5] = 0.0
    S[0, 1, 5, :len(vals)] = vals
    codes, scales = O.quantize_rows(S)
    assert scales[0, 1, 5] == np.float32(f)
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(ref["codes"], codes) and np.array_equal(ref["scale"], scales)
    assert np.array_equal(host(cg), codes)
    assert np.array_equal(host(sg), scales)


def test_prefill_requantizes_rows_whose_scale_rounds_to_zero():
    """A stored row with codes of at most 40 in magnitude and scale 2^-149
    (the smallest subnormal) carried through one window with alpha = 1,
    beta = 0: its values are unchanged, absmax / 127 is below half of 2^-149,
    so the window-end scale rounds to 0 and every code must be 0 (the codec
    reading: a row whose scale is 0 stores codes 0), as the oracle gives."""
    B, H, d, T = 1, 2, 128, 64
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=33)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    S = (np.random.default_rng(34).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    codes, scales = O.quantize_rows(S)
    rng = np.random.default_rng(35)
    codes[0, 0, 7] = rng.integers(-40, 41, size=d).astype(np.int8)
    codes[0, 0, 7, 3] = 40
    scales[0, 0, 7] = np.float32(2.0 ** -149)
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, codes0=codes, scale0=scales)
    assert ref["scale"][0, 0, 7] == 0.0 and not ref["codes"][0, 0, 7].any()
    o, cg, sg = ops.prefill_chunked(*_inputs(x), init_codes=dev(codes), init_scales=dev(scales),
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(cg), ref["codes"])
    assert np.array_equal(host(sg), ref["scale"])


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
    assert_free_scales(host(sg), ref["scale"], f"prefill 5 windows init={init}")


@pytest.mark.parametrize("state_bits", [8, 4])
def test_prefill_rotated_teacher_forced_chunks(state_bits):
    """GDNQ_FLAG_WHT on the chunked prefill (reading R23: q and k rotated by
    H/sqrt(128) in fp32 and rounded to bf16): B=2, H=3, four chunks, one per
    call, each from the GPU's previous state, the first from a random state
    quantized in the rotated basis.  Teacher-forced stage by stage:
      * the rotated operands the kernels used (read back from the workspace)
        against the oracle's rotation and rounding: bitwise, except +-1 bf16
        step on <= 0.1% of the elements (the fp32 sums run in different
        orders, so a value on a bf16 rounding tie may round either way);
      * the recurrence on those same operands: outputs (fp32) within 1e-3,
        codes +-1 on <= 0.1%, scales within 1e-5."""
    B, H, d, T = 2, 3, 128, 256
    qmax = 127 if state_bits == 8 else 7
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=41)
    S = (np.random.default_rng(42).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    codes, scales = O.quantize_rows(O.gdnq_oracle.rotate(S, np.float32), qmax=qmax)

    def pack(c):
        if state_bits == 8:
            return c
        u = (c[..., 0::2].astype(np.int16) & 0xF) | ((c[..., 1::2].astype(np.int16) & 0xF) << 4)
        return u.astype(np.uint8).view(np.int8)

    def unpack(c):
        if state_bits == 8:
            return c
        u = c.view(np.uint8).astype(np.int16)
        lo, hi = u & 0xF, u >> 4
        return np.stack([np.where(lo > 7, lo - 16, lo), np.where(hi > 7, hi - 16, hi)], -1).reshape(
            c.shape[:-1] + (2 * c.shape[-1],)).astype(np.int8)

    rows = B * W * H
    for c in range(T // W):
        xs = {k: np.ascontiguousarray(v[:, c * W:(c + 1) * W]) for k, v in x.items()}
        q_, k_, v_, a_, b_ = _inputs(xs)
        need = ops.prefill_workspace_size(q_, v_, wht=True)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        o, cg, sg = ops.prefill_chunked(q_, k_, v_, a_, b_, init_codes=dev(pack(codes)), init_scales=dev(scales),
                                        wht=True, out_dtype=torch.float32, state_bits=state_bits, workspace=ws)
        torch.cuda.synchronize()
        # the rotated q and k are the last 2 * rows * 128 bf16 of the workspace
        rot = host(ws[need - 2 * rows * d * 2:]).view(np.uint16).reshape(2, B, W, H, d)
        qr, kr = (wl.bf16_to_f32(rot[i]) for i in range(2))
        for name, got, src in (("q", qr, xs["q"]), ("k", kr, xs["k"])):
            r32 = O.gdnq_oracle.rotate(src, np.float32)
            ref = O.round_bf16(r32)
            diff = got != ref
            assert np.mean(diff) <= 1e-3, f"chunk {c}: {name} rotated operands differ on {np.mean(diff):.3%}"
            # every element is a bf16 rounding (half a bf16 step) of a value within
            # fp32 summation error (2^-20 of the row's norm) of the oracle's rotation
            half = np.spacing(np.abs(r32)).astype(np.float64) * 2.0 ** 15
            tol = half + 2.0 ** -20 * np.linalg.norm(src, axis=-1, keepdims=True)
            assert np.all(np.abs(got.astype(np.float64) - r32) <= tol), f"chunk {c}: rotated {name} off"
        ref = O.prefill(qr, kr, xs["v"], xs["alpha"], xs["beta"], W=W, codes0=codes, scale0=scales, qmax=qmax)
        err = max_rel_err(host(o), ref["o"])
        assert err <= OUT_TOL_F32, f"chunk {c}: o max relative error {err:.3e}"
        assert_codes(unpack(host(cg)), ref["codes"], f"chunk {c} codes")
        assert_scales(host(sg), ref["scale"], f"chunk {c} scales")
        codes, scales = unpack(host(cg)), host(sg)


def test_prefill_rotated_free_running_and_rotation_invariance():
    """B=2, H=2, T=320 in one call with the rotation, from a zero state,
    against the oracle's rotation and recurrence run on its own (outputs
    2e-2, codes +-1 on <= 0.1%, scales within the free-running drift bound:
    rotated operands on a bf16 tie may round apart, see above); and the
    outputs agree with the unrotated call within 2e-2 (the rotation keeps
    S q, up to the bf16 rounding of the rotated operands and the different
    requantization basis)."""
    B, H, d, T = 2, 2, 128, 320
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=43)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), wht=True, out_dtype=torch.float32)
    o0, _, _ = ops.prefill_chunked(*_inputs(x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=W, rot=True, qk_bf16=True)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_BF16
    assert_codes(host(cg), ref["codes"], "final codes")
    assert_free_scales(host(sg), ref["scale"], "rotated prefill 5 windows")
    assert max_rel_err(host(o), host(o0)) <= OUT_TOL_BF16


@pytest.mark.parametrize("state_bits", [8, 4])
def test_prefill_d64_teacher_forced_chunks(state_bits):
    """d_k = d_v = 64 (the library runs it as a zero-padded d = 128 head):
    B=2, H=3, four chunks, one per call, each from the GPU's previous state,
    the first from a random stored state.  Outputs (fp32) within 1e-3,
    codes +-1 on <= 0.1%, scales 1e-5; guard zones around every output."""
    B, H, d, T = 2, 3, 64, 256
    qmax = 127 if state_bits == 8 else 7
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=45)
    S = (np.random.default_rng(46).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    S[1, 2, 7] = 0.0  # a zero row
    codes, scales = O.quantize_rows(S, qmax=qmax)

    def pack(c):
        if state_bits == 8:
            return c
        u = (c[..., 0::2].astype(np.int16) & 0xF) | ((c[..., 1::2].astype(np.int16) & 0xF) << 4)
        return u.astype(np.uint8).view(np.int8)

    def unpack(c):
        if state_bits == 8:
            return c
        u = c.view(np.uint8).astype(np.int16)
        lo, hi = u & 0xF, u >> 4
        return np.stack([np.where(lo > 7, lo - 16, lo), np.where(hi > 7, hi - 16, hi)], -1).reshape(
            c.shape[:-1] + (2 * c.shape[-1],)).astype(np.int8)

    cb = d * state_bits // 8
    for c in range(T // W):
        xs = {k: np.ascontiguousarray(v[:, c * W:(c + 1) * W]) for k, v in x.items()}
        o = Guarded((B, W, H, d), torch.float32)
        cg = Guarded((B, H, d, cb), torch.int8)
        sg = Guarded((B, H, d), torch.float32)
        ops.prefill_chunked(*_inputs(xs), init_codes=dev(pack(codes)), init_scales=dev(scales),
                            out_dtype=torch.float32, o=o.t, codes=cg.t, scales=sg.t, state_bits=state_bits)
        torch.cuda.synchronize()
        assert o.guards_intact() and cg.guards_intact() and sg.guards_intact()
        ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W, codes0=codes, scale0=scales,
                        qmax=qmax)
        err = max_rel_err(host(o.t), ref["o"])
        assert err <= OUT_TOL_F32, f"chunk {c}: o max relative error {err:.3e}"
        assert_codes(unpack(host(cg.t)), ref["codes"], f"chunk {c} codes")
        assert_scales(host(sg.t), ref["scale"], f"chunk {c} scales")
        codes, scales = unpack(host(cg.t)), host(sg.t)


def test_prefill_d64_single_head_from_zero():
    """The single-head d = 64 recurrence of the parity workload (q, k
    L2-normalized, fp32 inputs rounded to bf16 for the prefill), 256 tokens
    from a zero state in one call with bf16 output: free-running against the
    oracle (outputs 2e-2, final codes +-1 on <= 0.1%)."""
    x = wl.single_head_fp32(T=256, d=64, seed=0)
    xs = {n: wl.bf16_round(x[n])[None, :, None] for n in ("q", "k", "v")}
    xs.update({n: x[n][None, :, None] for n in ("alpha", "beta")})
    o, cg, sg = ops.prefill_chunked(*_inputs(xs), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W)
    assert max_rel_err(host(o), ref["o"]) <= OUT_TOL_BF16
    assert_codes(host(cg), ref["codes"], "final codes")
    assert_free_scales(host(sg), ref["scale"], "d = 64 single head, 4 windows")


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


def test_prefill_batch4_seq8192_heads16_every_window_teacher_forced():
    """The prefill workload at its full size (B=4, T=8192, H=16, d=128,
    chunk = window = 64) in one call, as it is timed (bf16 output), and the
    same tokens again one window per call, each call from the state the
    previous one left on the GPU.

    * The window-per-call run ends in the one-call run's codes and scales,
      bitwise, and its outputs round to the one-call bf16 outputs: so the
      checks below are checks of the timed call.
    * Every one of the 128 windows, on all 64 (sequence, head) pairs, is
      compared with the oracle started from the GPU's state before that
      window (teacher-forced): outputs (fp32) within 1e-3, requantized
      codes +-1 on <= 0.1%, scales within 1e-5."""
    B, T, H, d = 4, 8192, 16, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=0)
    q, k, v, a, b = _inputs(x)
    o_all, c_all, s_all = ops.prefill_chunked(q, k, v, a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_all_h = host(o_all)
    assert np.isfinite(o_all_h).all()
    codes = torch.zeros((B, H, d, d), dtype=torch.int8, device=DEV)
    scales = torch.zeros((B, H, d), dtype=torch.float32, device=DEV)
    ws = torch.empty(ops.prefill_workspace_size(q[:, :W], v[:, :W]), dtype=torch.uint8, device=DEV)
    jobs = []
    with oracle_pool.pool() as ex:
        for c in range(T // W):
            sl = slice(c * W, (c + 1) * W)
            before_c, before_s = host(codes), host(scales)
            cn = torch.empty_like(codes)
            sn = torch.empty_like(scales)
            o, _, _ = ops.prefill_chunked(q[:, sl].contiguous(), k[:, sl].contiguous(),
                                          v[:, sl].contiguous(), a[:, sl].contiguous(),
                                          b[:, sl].contiguous(), init_codes=codes, init_scales=scales,
                                          codes=cn, scales=sn, out_dtype=torch.float32, workspace=ws)
            torch.cuda.synchronize()
            go = host(o)
            # the one-call bf16 outputs are these fp32 outputs rounded once
            ob = o_all_h[:, sl]
            assert np.all(np.abs(ob - go) <= np.abs(go) * 2.0 ** -8 + 1e-30), f"window {c}: bf16 outputs"
            xs = {n: np.ascontiguousarray(x[n][:, sl]) for n in ("q", "k", "v", "alpha", "beta")}
            fut = oracle_pool.submit(ex, "prefill_window", xs, before_c, before_s, W, 127)
            jobs.append((c, fut, go, host(cn), host(sn)))
            codes, scales = cn, sn
        assert torch.equal(codes, c_all) and torch.equal(scales, s_all)
        worst_o = worst_flip = 0.0
        for c, fut, go, gc, gs in jobs:
            ro, rc, rs = fut.result()
            err = max_rel_err(go, ro)
            assert err <= OUT_TOL_F32, f"window {c}: o max relative error {err:.3e}"
            worst_o = max(worst_o, err)
            worst_flip = max(worst_flip, assert_codes(gc, rc, f"window {c} codes"))
            assert_scales(gs, rs, f"window {c} scales")
    print(f"B4 T8192 H16: 128 windows x 64 heads teacher-forced, worst o {worst_o:.2e}, "
          f"worst flip fraction {worst_flip:.2e}")


def test_prefill_batch4_seq8192_heads16_free_running_sampled():
    """Diagnostic beside the gate above: three sampled (sequence, head) pairs
    of the full-size call followed by the oracle on its own over all 8192
    tokens (128 windows).  Outputs within 2e-2 and final codes +-1 on
    <= 0.1%; scales within the free-running drift bound of two code units
    relative (2/127): once an admitted +-1 difference exists the two runs
    carry different states, so the per-requantization scale bar does not
    apply (the design notes derive the bound)."""
    B, T, H, d = 4, 8192, 16, 128
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=d, dv=d, seed=0)
    o, cg, sg = ops.prefill_chunked(*_inputs(x), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    go, gc, gs = host(o), host(cg), host(sg)
    for b, h in ((0, 0), (2, 7), (3, 15)):
        xs = {k: np.ascontiguousarray(v[b:b + 1, :, h:h + 1]) for k, v in x.items()}
        ref = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W)
        err = max_rel_err(go[b, :, h], ref["o"][0, :, 0])
        assert err <= OUT_TOL_BF16, f"(b={b}, h={h}) o error {err:.3e}"
        assert_codes(gc[b, h], ref["codes"][0, 0], f"(b={b}, h={h}) codes")
        assert_free_scales(gs[b, h], ref["scale"][0, 0], f"prefill 128 windows (b={b}, h={h})")
