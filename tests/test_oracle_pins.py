"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test names the mistake it would catch.  None of them re-types the
oracle's own formula: they use hand-derived values (tests/golden), closed
forms, invariants and special cases.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as wl
from conftest import read_golden

F32, F64 = np.float32, np.float64


def _rows(s):
    return np.array([[float(Fraction(x)) for x in r.split()] for r in s.split("|")])


# ---------------------------------------------------------------- codec
def test_codec_golden_rows():
    """Hand-derived rows: scale = absmax/127, round-half-even ties, zero row.
    Catches /128 instead of /127, round-half-away, missing abs, missing clamp."""
    g = read_golden("codec_rows.txt")
    for row, sc, cd in zip(g["row"], g["scale"], g["codes"]):
        x = np.array([float(v) for v in row.split()], F32)[None]
        codes, scale = O.quantize_rows(x)
        assert scale[0] == F32(float(sc))
        assert codes.dtype == np.int8
        assert codes[0].tolist() == [int(v) for v in cd.split()]


def test_codec_subnormal_scale_golden():
    """A row whose scale is an fp32 subnormal (2^-140, beyond the range where
    1/scale is finite): the codes are the exact quotients.  Catches a codec
    that multiplies by a reciprocal, or that flushes subnormals to zero."""
    g = read_golden("codec_subnormal.txt")
    for p2, row, sc, cd in zip(g["pow2"], g["row"], g["scale"], g["codes"]):
        f = 2.0 ** int(p2)
        x = (np.array([float(v) for v in row.split()], F64) * f).astype(F32)[None]
        assert np.array_equal(x[0].astype(F64), np.array([float(v) for v in row.split()]) * f)  # exact
        codes, scale = O.quantize_rows(x)
        assert scale[0] == F32(float(sc) * f) and scale[0] < np.finfo(F32).tiny
        assert codes[0].tolist() == [int(v) for v in cd.split()]


def test_codec_properties_random():
    """P4: |x - deq(quant(x))| <= scale/2 per entry; every nonzero row reaches
    |code| = 127; quant(-x) = -quant(x); codes in [-127, 127]."""
    g = np.random.default_rng(1)
    x = (g.standard_normal((500, 128)) * np.exp(g.uniform(-8, 8, (500, 1)))).astype(F32)
    x[7] = 0.0
    codes, scale = O.quantize_rows(x)
    deq = O.dequantize(codes, scale, F64)
    err = np.abs(x.astype(F64) - deq)
    assert np.all(err <= scale[:, None].astype(F64) * (0.5 + 1e-6) + 1e-30)
    nz = scale > 0
    assert np.all(np.max(np.abs(codes[nz].astype(int)), axis=1) == 127)
    assert np.all(codes[7] == 0) and scale[7] == 0
    c2, s2 = O.quantize_rows(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)
    assert codes.min() >= -127 and codes.max() <= 127


def test_codec_decision_in_fp32_for_fp64_input():
    """The codec takes its decision in fp32 whatever the working precision."""
    g = np.random.default_rng(2)
    x = g.standard_normal((10, 64))
    c64, s64 = O.quantize_rows(x)
    c32, s32 = O.quantize_rows(x.astype(F32))
    assert np.array_equal(c64, c32) and np.array_equal(s64, s32)


# ---------------------------------------------------------------- WHT
def test_wht_sylvester4_golden():
    g = read_golden("sylvester4.txt")
    H4 = np.array([[float(v) for v in r.split()] for r in g["row"]])
    assert np.array_equal(O.wht_matrix(4) * 2.0, H4)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_wht_orthogonal_symmetric(d):
    H = O.wht_matrix(d)
    assert np.allclose(H @ H.T, np.eye(d), atol=1e-13)
    assert np.array_equal(H, H.T)
    e0 = np.zeros(d)
    e0[0] = 1
    assert np.allclose(H @ e0, np.full(d, 1 / np.sqrt(d)), atol=1e-15)
    # recursive Sylvester structure H_2d = [[H, H], [H, -H]] / sqrt(2)
    if d >= 4:
        h = O.wht_matrix(d // 2)
        top = np.hstack([h, h])
        bot = np.hstack([h, -h])
        assert np.allclose(np.vstack([top, bot]) / np.sqrt(2), H, atol=1e-15)


# ---------------------------------------------------------------- worked example
def _worked():
    g = read_golden("gdn_worked_example.txt")
    W = int(g["W"][0])
    q = _rows(g["q"][0])
    k = _rows(g["k"][0])
    v = _rows(g["v"][0])
    a = np.array([float(x) for x in g["alpha"][0].split()])
    b = np.array([float(x) for x in g["beta"][0].split()])
    o = _rows(g["o"][0])
    c2 = _rows(g["codes_after_t2"][0]).astype(int)
    s2 = np.array([float(Fraction(x)) for x in g["scale_after_t2"][0].split()])
    cf = _rows(g["codes_final"][0]).astype(int)
    sf_txt = g["scale_final"][0].split()
    sf = np.array([F32(0.25), F32(16) / F32(127)], F32)
    assert sf_txt == ["0.25", "16/127"]
    return W, q, k, v, a, b, o, c2, s2, cf, sf


@pytest.mark.parametrize("dtype", [F32, F64])
def test_worked_example_exact(dtype):
    """Hand-derived 2x2 example: catches the decay applied after the erase,
    a transposed write (k v^T), output taken after requantization, a window
    closing one token late or early, and round-half-away at the -63.5 tie."""
    W, q, k, v, a, b, o, c2, s2, cf, sf = _worked()
    r2 = O.run_windowed(q[:2, None], k[:2, None], v[:2, None], a[:2, None], b[:2, None],
                        W=W, dtype=dtype)
    assert np.array_equal(r2["codes"][0], c2)
    assert np.array_equal(r2["scale"][0], s2.astype(F32))
    r = O.run_windowed(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None],
                       W=W, dtype=dtype)
    assert np.array_equal(r["o"][:, 0], o.astype(dtype))
    assert np.array_equal(r["codes"][0], cf)
    assert np.array_equal(r["scale"][0], sf)
    assert r["n"] == 0


def test_worked_example_via_decode_steps():
    """P11 on the worked example: four single-token decode calls that carry
    (codes, scales, buffer, fill) reproduce the one-shot run exactly."""
    W, q, k, v, a, b, o, c2, s2, cf, sf = _worked()
    codes = np.zeros((1, 1, 2, 2), np.int8)
    scales = np.zeros((1, 1, 2), F32)
    bk = np.full((1, 1, W, 2), np.nan, F32)
    bv = np.full((1, 1, W, 2), np.nan, F32)
    ba = np.full((1, 1, W), np.nan, F32)
    bb = np.full((1, 1, W), np.nan, F32)
    fill = np.zeros(1, np.int32)
    for t in range(4):
        out = O.decode_step(q[t][None, None], k[t][None, None], v[t][None, None],
                            a[t:t + 1][None], b[t:t + 1][None], codes, scales,
                            bk, bv, ba, bb, fill, W)
        ot, codes, scales, bk, bv, ba, bb, fill = out
        assert np.array_equal(ot[0, 0], o[t].astype(F32))
    assert np.array_equal(codes[0, 0], cf)
    assert np.array_equal(scales[0, 0], sf)


# ---------------------------------------------------------------- recurrence pins
def _rand_state(g, N, dv, dk):
    S = (g.standard_normal((N, dv, dk)) * 0.5).astype(F32)
    return O.quantize_rows(S)


def _unit(x, dtype):
    x = x.astype(dtype)
    return (x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))).astype(dtype)


def _rand_tokens(g, T, N, dk, dv, dtype=F32):
    q = _unit(g.standard_normal((T, N, dk)), dtype)
    k = _unit(g.standard_normal((T, N, dk)), dtype)
    v = g.standard_normal((T, N, dv)).astype(dtype)
    a = g.uniform(0.9, 0.999, (T, N)).astype(dtype)
    b = g.uniform(0, 1, (T, N)).astype(dtype)
    return q, k, v, a, b


@pytest.mark.parametrize("W", [None, 1, 3, 8])
@pytest.mark.parametrize("rot", [False, True])
def test_p2_unit_beta_reads_back_v(W, rot):
    """P2: beta = 1, ||k|| = 1, q = k  =>  o_t = v_t for any state, fill and
    window position.  Catches a dropped erase term, a wrong sign in it, the
    wrong key in the erase and the decay applied to the write."""
    g = np.random.default_rng(3)
    T, N, d = 11, 3, 16
    q, k, v, a, b = _rand_tokens(g, T, N, d, d, F64)
    b[:] = 1.0
    codes, scale = _rand_state(g, N, d, d)
    buf = {"k": _unit(g.standard_normal((2, N, d)), F64),
           "v": g.standard_normal((2, N, d)), "alpha": g.uniform(0.9, 1, (2, N)),
           "beta": g.uniform(0, 1, (2, N))}
    r = O.run_windowed(k, k, v, a, b, W=W, codes0=codes, scale0=scale,
                       buffer0=buf if W != 1 else None, rot=rot, dtype=F64)
    assert np.max(np.abs(r["o"] - v)) < 1e-12


def test_p2_exact_fp32_basis_keys():
    """P2 in fp32 with exact arithmetic: basis keys, integer state and values."""
    d = 8
    S0 = np.arange(-32, 32, dtype=F32).reshape(d, d)  # |x| <= 32 integer
    codes, scale = O.quantize_rows(S0 * (127 / 32.0))
    T = 6
    k = np.eye(d, dtype=F32)[[3, 1, 4, 1, 5, 0]][:, None]
    v = np.array([[5, -3, 2, 7, 0, 1, -8, 4]] * T, F32)[:, None] * np.arange(1, T + 1)[:, None, None]
    a = np.full((T, 1), 0.5, F32)
    b = np.ones((T, 1), F32)
    r = O.run_windowed(k, k, v.astype(F32), a, b, W=4, codes0=codes[None], scale0=scale[None])
    assert np.array_equal(r["o"], v.astype(F32))


def test_p3_identity_transition_keeps_state():
    """P3: alpha = 1, beta = 0 leaves the state unchanged; requantization is
    idempotent on codes (scales may move by one ulp)."""
    g = np.random.default_rng(4)
    T, N, d = 9, 4, 16
    q, k, v, a, b = _rand_tokens(g, T, N, d, d)
    a[:] = 1
    b[:] = 0
    codes, scale = _rand_state(g, N, d, d)
    r = O.run_windowed(q, k, v, a, b, W=3, codes0=codes, scale0=scale)
    assert np.array_equal(r["codes"], codes)
    ulp = np.spacing(scale)
    assert np.all(np.abs(r["scale"] - scale) <= ulp)
    S = O.dequantize(codes, scale, F64)
    o_ref = np.einsum("nrc,tnc->tnr", S, q.astype(F64))
    assert np.allclose(r["o"], o_ref, rtol=1e-5, atol=1e-6)


def test_p8_basis_keys_exact_state():
    """P8: alpha = beta = 1 and distinct basis keys e_pi(t) give
    S = sum_t v_t e_pi(t)^T exactly; with row max 127 the scale is 1 and the
    codes equal the values."""
    d = 8
    perm = [5, 2, 7, 0, 3, 6, 1, 4]
    k = np.eye(d, dtype=F32)[perm][:, None]
    g = np.random.default_rng(5)
    v = g.integers(-126, 127, (d, d)).astype(F32)
    v[perm.index(0)] = 127.0  # column 0 of S holds 127 in every row
    v = v[:, None]
    a = np.ones((d, 1), F32)
    b = np.ones((d, 1), F32)
    r = O.run_windowed(k, k, v, a, b, W=d)
    S_exp = np.zeros((d, d), F32)
    for t, p in enumerate(perm):
        S_exp[:, p] = v[t, 0]
    assert np.array_equal(r["scale"][0], np.ones(d, F32))
    assert np.array_equal(r["codes"][0].astype(F32), S_exp)


def test_p9_pure_decay_is_exact_power_of_two():
    """P9: beta = 0, alpha = 1/2: S_T = 2^-T S_0 exactly, codes unchanged
    across windows, scales times 2^-W per window."""
    g = np.random.default_rng(6)
    T, N, d, W = 8, 3, 16, 4
    q, k, v, a, b = _rand_tokens(g, T, N, d, d)
    a[:] = 0.5
    b[:] = 0
    codes, scale = _rand_state(g, N, d, d)
    r = O.run_windowed(q, k, v, a, b, W=W, codes0=codes, scale0=scale)
    assert np.array_equal(r["codes"], codes)
    assert np.array_equal(r["scale"], (scale * F32(2.0 ** -T)).astype(F32))
    r1 = O.run_windowed(q[:W], k[:W], v[:W], a[:W], b[:W], W=W, codes0=codes, scale0=scale)
    assert np.array_equal(r1["scale"], (scale * F32(2.0 ** -W)).astype(F32))


def test_p12_row_norm_non_expansive():
    """P12: beta in [0,1], ||k|| = 1: ||S_t[r]|| <= alpha ||S_{t-1}[r]|| + beta |v[r]|."""
    g = np.random.default_rng(7)
    N, d = 5, 32
    S = g.standard_normal((N, d, d))
    for _ in range(20):
        q, k, v, a, b = _rand_tokens(g, 1, N, d, d, F64)
        S2 = O.gdn_step(S, k[0], v[0], a[0], b[0])
        lhs = np.linalg.norm(S2, axis=-1)
        rhs = a[0][:, None] * np.linalg.norm(S, axis=-1) + b[0][:, None] * np.abs(v[0])
        assert np.all(lhs <= rhs + 1e-12)
        S = S2


def test_p13_linear_in_v():
    """P13: with no quantization and zero initial state, o is linear in v."""
    g = np.random.default_rng(8)
    T, N, d = 10, 2, 8
    q, k, v, a, b = _rand_tokens(g, T, N, d, d, F64)
    v2 = g.standard_normal(v.shape)
    o1 = O.run_windowed(q, k, v, a, b, W=None, dtype=F64)["o"]
    o2 = O.run_windowed(q, k, v2, a, b, W=None, dtype=F64)["o"]
    o3 = O.run_windowed(q, k, 2.5 * v - 0.75 * v2, a, b, W=None, dtype=F64)["o"]
    assert np.max(np.abs(o3 - (2.5 * o1 - 0.75 * o2))) < 1e-12


def test_p1_window_never_closing_is_unquantized():
    """P1: from a zero state, a window that never closes (W > T) gives exactly
    the unquantized recurrence (no requantization happens)."""
    g = np.random.default_rng(9)
    T, N, d = 12, 3, 16
    q, k, v, a, b = _rand_tokens(g, T, N, d, d)
    r_inf = O.run_windowed(q, k, v, a, b, W=None)
    r_big = O.run_windowed(q, k, v, a, b, W=T + 1)
    assert np.array_equal(r_inf["o"], r_big["o"])
    assert r_big["n"] == T and np.all(r_big["codes"] == 0)


def test_p6_window_of_one_and_window_of_t():
    """P6: W = 1 requantizes after every token; W = T quantizes only at the end."""
    g = np.random.default_rng(10)
    T, N, d = 6, 2, 8
    q, k, v, a, b = _rand_tokens(g, T, N, d, d)
    r1 = O.run_windowed(q, k, v, a, b, W=1)
    S = np.zeros((N, d, d), F32)
    for t in range(T):
        S = O.gdn_step(S, k[t], v[t], a[t], b[t])
        ot = np.matmul(S, q[t][..., None])[..., 0]
        assert np.array_equal(r1["o"][t], ot)
        c, s = O.quantize_rows(S)
        S = O.dequantize(c, s)
    rT = O.run_windowed(q, k, v, a, b, W=T)
    rinf = O.run_windowed(q, k, v, a, b, W=None)
    assert np.array_equal(rT["o"], rinf["o"])
    c, s = O.quantize_rows(rinf["S"])
    assert np.array_equal(rT["codes"], c) and np.array_equal(rT["scale"], s)


@pytest.mark.parametrize("W", [None, 8, 16])
def test_p5_chunked_equals_sequential_fp64(W):
    """P5: the chunkwise (UT/WY) form equals the token-by-token recurrence.
    Catches errors in either: a wrong decay ratio, A on the wrong side of the
    diagonal, a missing beta."""
    g = np.random.default_rng(11)
    T, d, C = 32, 16, 8
    q, k, v, a, b = _rand_tokens(g, T, 1, d, d, F64)
    seq = O.run_windowed(q, k, v, a, b, W=W, dtype=F64)
    ch = O.chunked_fp64(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], C=C, W=W)
    assert np.max(np.abs(seq["o"][:, 0] - ch["o"])) < 1e-10 * max(1, np.abs(seq["o"]).max())
    if W is None:
        assert np.max(np.abs(seq["S"][0] - ch["S"])) < 1e-10
    else:
        diff = np.abs(seq["codes"][0].astype(int) - ch["codes"].astype(int))
        assert diff.max() <= 1 and diff.mean() < 0.01


def test_p5_chunked_with_initial_state():
    g = np.random.default_rng(12)
    T, d, C = 24, 8, 8
    q, k, v, a, b = _rand_tokens(g, T, 1, d, d, F64)
    S0 = g.standard_normal((d, d))
    c0, s0 = O.quantize_rows(S0)
    seq = O.run_windowed(q, k, v, a, b, W=None, codes0=c0[None], scale0=s0[None], dtype=F64)
    ch = O.chunked_fp64(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], C=C,
                        S0=O.dequantize(c0, s0, F64))
    assert np.max(np.abs(seq["o"][:, 0] - ch["o"])) < 1e-10


@pytest.mark.parametrize("with_s0", [False, True])
def test_p10_ssd_closed_form(with_s0):
    """P10: the scalar-decay SSD recurrence equals its quadratic closed form and
    its chunked form."""
    g = np.random.default_rng(13)
    T, dk, dv, C = 24, 8, 4, 8
    q = g.standard_normal((T, 1, dk))
    k = g.standard_normal((T, 1, dk))
    v = g.standard_normal((T, 1, dv))
    a = np.exp(-np.log1p(np.exp(-3 + 0.5 * g.standard_normal((T, 1)))))
    S0 = g.standard_normal((dv, dk)) if with_s0 else None
    c0 = s0 = None
    if with_s0:
        c0, s0 = O.quantize_rows(S0)
        S0 = O.dequantize(c0, s0, F64)
    seq = O.run_windowed(q, k, v, a, None, W=None, kind="ssd", dtype=F64,
                         codes0=None if c0 is None else c0[None],
                         scale0=None if s0 is None else s0[None])
    cf = O.ssd_closed_form(q[:, 0], k[:, 0], v[:, 0], a[:, 0], S0=S0)
    assert np.max(np.abs(seq["o"][:, 0] - cf)) < 1e-10
    ch = O.chunked_fp64(q[:, 0], k[:, 0], v[:, 0], a[:, 0], C=C, kind="ssd", S0=S0)
    assert np.max(np.abs(ch["o"] - cf)) < 1e-10
    assert np.max(np.abs(ch["S"] - seq["S"][0])) < 1e-10


def test_p7_rotation_invariance():
    """P7: rotating q and k by the normalised WHT leaves o unchanged and turns
    the state into S H (unquantized, fp64)."""
    g = np.random.default_rng(14)
    T, N, d = 10, 2, 16
    q, k, v, a, b = _rand_tokens(g, T, N, d, d, F64)
    r0 = O.run_windowed(q, k, v, a, b, W=None, dtype=F64)
    r1 = O.run_windowed(q, k, v, a, b, W=None, rot=True, dtype=F64)
    assert np.max(np.abs(r0["o"] - r1["o"])) < 1e-12
    H = O.wht_matrix(d)
    assert np.max(np.abs(r1["S"] - r0["S"] @ H)) < 1e-12
    # SSD as well
    s0 = O.run_windowed(q, k, v, a, None, W=None, kind="ssd", dtype=F64)
    s1 = O.run_windowed(q, k, v, a, None, W=None, kind="ssd", rot=True, dtype=F64)
    assert np.max(np.abs(s0["o"] - s1["o"])) < 1e-12


def test_rotated_operands_rounded_to_bf16_golden():
    """The GDN prefill's rotated operands (reading R23: rotate in fp32, round
    to bf16), by hand: H e0 / sqrt(128) has every entry 2^-3.5 =
    0.0883883..., whose nearest bf16 is 181/2048 = 0.08837890625 (8
    significant bits: 1.41421 x 128 = 181.02 -> 181); H (e0 + e1) / sqrt(128)
    has 2^-2.5 = 0.1767767 on even indices, nearest bf16 181/1024, and 0 on
    odd ones.  Catches rounding before the rotation and a missing 1/sqrt(d)."""
    d = 128
    x = np.zeros((2, d), F32)
    x[0, 0] = 1.0
    x[1, 0] = x[1, 1] = 1.0
    q, k = O.gdnq_oracle._prepare_qk(x, x, True, False, F32, qk_bf16=True)
    assert np.all(k[0] == F32(181 / 2048)) and np.all(q[0] == F32(181 / 2048))
    assert np.all(k[1, 0::2] == F32(181 / 1024)) and np.all(k[1, 1::2] == 0)
    q0, _ = O.gdnq_oracle._prepare_qk(x, x, True, False, F32)
    assert np.all(np.abs(q0[0] - F32(2 ** -3.5)) <= 2e-8)


def test_qk_int8_operands_within_half_scale():
    """Int8 operand quantization of rotated q, k: every operand entry moves by
    at most half its row scale, and the run equals one on pre-quantized inputs."""
    g = np.random.default_rng(15)
    T, N, dk, dv = 6, 2, 16, 8
    q = g.standard_normal((T, N, dk))
    k = g.standard_normal((T, N, dk))
    v = g.standard_normal((T, N, dv))
    a = g.uniform(0.9, 1, (T, N))
    r = O.run_windowed(q, k, v, a, None, W=None, kind="ssd", rot=True, qk_int8=True, dtype=F64)
    H = O.wht_matrix(dk)
    kr = k @ H.T
    ck, sk = O.quantize_rows(kr)
    kq = O.dequantize(ck, sk, F64)
    assert np.all(np.abs(kq - kr) <= sk[..., None] * (0.5 + 1e-6))
    cq, sq = O.quantize_rows(q @ H.T)
    r2 = O.run_windowed(O.dequantize(cq, sq, F64), kq, v, a, None, W=None, kind="ssd", dtype=F64)
    assert np.max(np.abs(r["o"] - r2["o"])) < 1e-12


# ---------------------------------------------------------------- decode protocol
def test_p14_sweep_equals_replay():
    """P14: the backward sweep (decode design) equals the replay, random fills."""
    g = np.random.default_rng(16)
    d = 16
    for f in [0, 1, 5, 15]:
        codes, scale = _rand_state(g, 1, d, d)
        bq, bk, bv, ba, bb = _rand_tokens(g, f + 1, 1, d, d, F64)
        buf = {"k": bk[:f], "v": bv[:f], "alpha": ba[:f], "beta": bb[:f]}
        r = O.run_windowed(bq[f:], bk[f:], bv[f:], ba[f:], bb[f:], W=None, codes0=codes,
                           scale0=scale, buffer0=buf, dtype=F64)
        o = O.sweep_mirror(bq[f, 0], bk[f, 0], bv[f, 0], ba[f, 0], bb[f, 0], codes[0], scale[0],
                           bk[:f, 0], bv[:f, 0], ba[:f, 0], bb[:f, 0])
        assert np.max(np.abs(o - r["o"][0, 0])) < 1e-12


def test_p11_one_run_equals_decode_calls_and_resume():
    """P11: T tokens in one run equal T decode calls carrying (codes, scales,
    buffer, fill); a save/restore half way is bitwise; prefill + decode equals
    one run."""
    g = np.random.default_rng(17)
    B, H, d, W, T = 2, 2, 8, 4, 11
    q, k, v, a, b = _rand_tokens(g, T, B * H, d, d)
    r = O.run_windowed(q, k, v, a, b, W=W)
    codes = np.zeros((B, H, d, d), np.int8)
    scales = np.zeros((B, H, d), F32)
    bk = np.full((B, H, W, d), np.nan, F32)
    bv = np.full((B, H, W, d), np.nan, F32)
    ba = np.full((B, H, W), np.nan, F32)
    bb = np.full((B, H, W), np.nan, F32)
    fill = np.zeros(B, np.int32)
    snap = None
    rs = lambda x: x.reshape((B, H) + x.shape[1:])  # noqa: E731
    for t in range(T):
        if t == 5:
            snap = [np.copy(x) for x in (codes, scales, bk, bv, ba, bb, fill)]
            codes, scales, bk, bv, ba, bb, fill = [np.copy(x) for x in snap]
        out = O.decode_step(rs(q[t]), rs(k[t]), rs(v[t]), rs(a[t]), rs(b[t]), codes, scales,
                            bk, bv, ba, bb, fill, W)
        ot, codes, scales, bk, bv, ba, bb, fill = out
        assert np.array_equal(ot.reshape(B * H, d), r["o"][t])
    assert np.array_equal(codes.reshape(B * H, d, d), r["codes"])
    assert np.array_equal(scales.reshape(B * H, d), r["scale"])
    assert np.all(fill == T % W)
    # prefill of the first 8 tokens (two whole windows) then decode of 3
    qq = lambda x: np.moveaxis(x.reshape((T, B, H) + x.shape[2:]), 0, 1)  # noqa: E731
    p = O.prefill(qq(q)[:, :8], qq(k)[:, :8], qq(v)[:, :8], qq(a)[:, :8], qq(b)[:, :8], W=W)
    assert p["n"] == 0
    codes, scales = p["codes"], p["scale"]
    bk[:] = np.nan
    fill = np.zeros(B, np.int32)
    for t in range(8, T):
        out = O.decode_step(rs(q[t]), rs(k[t]), rs(v[t]), rs(a[t]), rs(b[t]), codes, scales,
                            bk, bv, ba, bb, fill, W)
        ot, codes, scales, bk, bv, ba, bb, fill = out
        assert np.array_equal(ot.reshape(B * H, d), r["o"][t])


def test_decode_buffer_is_the_window_and_poison_is_not_read():
    """The decode call reads only buffer slots < fill (NaN poison elsewhere)
    and appends the token's write at slot fill."""
    d = wl.decode_batch(B=4, H=2, dk=16, dv=16, W=8, seed=3)
    codes, scales = O.quantize_rows(d["state"])
    out = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], codes, scales,
                        d["buf_k"], d["buf_v"], d["buf_alpha"], d["buf_beta"], d["fill"], 8)
    o, c2, s2, bk, bv, ba, bb, fill_out = out
    assert np.all(np.isfinite(o))
    assert np.array_equal(fill_out, (d["fill"] + 1) % 8)
    for bi in range(4):
        f = d["fill"][bi]
        if f + 1 < 8:
            assert np.array_equal(bk[bi, :, f], d["k"][bi])
            assert np.array_equal(bb[bi, :, f], d["beta"][bi])
            assert np.array_equal(c2[bi], codes[bi])
        else:
            assert np.all(np.isfinite(s2[bi]))


# ---------------------------------------------------------------- bf16 window buffer (variant)
def test_round_bf16_golden():
    """Round-to-nearest-even onto bf16, values worked by hand from the bit
    patterns: exact ties go to the even neighbour, a carry can reach the
    exponent, bf16 values are fixed points."""
    cases = [
        (1.0, 1.0),
        (1.0 + 2.0 ** -8, 1.0),                      # 0x3F808000: tie, kept LSB 0 -> down
        (1.0 + 3 * 2.0 ** -8, 1.015625),             # 0x3F818000: tie, kept LSB 1 -> up
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0078125),   # just above the tie -> up
        (-2.5, -2.5),                                # already bf16
        (np.float32(np.pi), 3.140625),               # 0x40490FDB -> 0x40490000
        (np.uint32(0x3FFFFFFF).view(F32), 2.0),      # carry into the exponent
        (0.0, 0.0),
    ]
    x = np.array([c[0] for c in cases], F32)
    want = np.array([c[1] for c in cases], F32)
    assert np.array_equal(O.round_bf16(x), want)


def test_round_bf16_matches_torch_cast():
    """The same rounding as torch's fp32 -> bfloat16 cast (a library routine)."""
    import torch
    g = np.random.default_rng(31)
    x = (g.standard_normal(4096) * np.exp(g.uniform(-20, 20, 4096))).astype(F32)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.round_bf16(x), t)


def test_buf_bf16_lossless_for_bf16_inputs():
    """Without rotation, bf16 inputs make the bf16 buffer lossless: every
    output of a step (o, codes, scales, buffers, fill) equals the fp32-buffer
    step bit for bit, over several steps and a window close."""
    W = 6
    d = wl.decode_batch(B=3, H=2, dk=16, dv=16, W=W, seed=5, fill=np.array([0, 3, 5]), poison=False)
    codes, scales = O.quantize_rows(d["state"])
    bufs = [O.round_bf16(d["buf_k"]), O.round_bf16(d["buf_v"]), d["buf_alpha"], d["buf_beta"]]
    st32 = [codes, scales] + [np.copy(x) for x in bufs] + [d["fill"]]
    st16 = [codes, scales] + [np.copy(x) for x in bufs] + [d["fill"]]
    for t in range(8):
        x = wl.decode_tokens(B=3, H=2, dk=16, dv=16, step=t, seed=6)
        a = O.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *st32[:6], st32[6], W)
        b = O.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *st16[:6], st16[6], W,
                          buf_bf16=True)
        for u, w in zip(a, b):
            assert np.array_equal(u, w, equal_nan=True)
        st32, st16 = list(a[1:]), list(b[1:])


def test_buf_bf16_rotated_write_is_rounded_when_stored():
    """With rotation the rotated key is not a bf16 value: the step's own
    output uses it exactly (same as the fp32 buffer), the stored copy is its
    bf16 rounding, and the next step replays the rounded copy."""
    W = 8
    d = wl.decode_batch(B=2, H=2, dk=16, dv=16, W=W, seed=7, fill=np.array([1, 2]), poison=False)
    codes, scales = O.quantize_rows(d["state"])
    bk, bv = O.round_bf16(d["buf_k"]), O.round_bf16(d["buf_v"])
    args = (codes, scales, bk, bv, d["buf_alpha"], d["buf_beta"], d["fill"], W)
    a = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], *args, rot=True)
    b = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], *args, rot=True, buf_bf16=True)
    assert np.array_equal(a[0], b[0])
    for s_ in range(2):
        f = int(d["fill"][s_])
        assert np.array_equal(b[3][s_, :, f], O.round_bf16(a[3][s_, :, f]))
        assert np.array_equal(b[4][s_, :, f], O.round_bf16(a[4][s_, :, f]))
        assert not np.array_equal(b[3][s_, :, f], a[3][s_, :, f])
    # the next step from the bf16-buffer state equals a replay of the rounded writes
    x = wl.decode_tokens(B=2, H=2, dk=16, dv=16, step=1, seed=8)
    c = O.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *b[1:7], b[7], W, rot=True,
                      buf_bf16=True)
    for s_ in range(2):
        f = int(b[7][s_])
        buf = {"k": np.moveaxis(b[3][s_, :, :f], 1, 0), "v": np.moveaxis(b[4][s_, :, :f], 1, 0),
               "alpha": b[5][s_, :, :f].T, "beta": b[6][s_, :, :f].T}
        r = O.run_windowed(x["q"][s_][None], x["k"][s_][None], x["v"][s_][None],
                           x["alpha"][s_][None], x["beta"][s_][None], W=W, codes0=b[1][s_],
                           scale0=b[2][s_], buffer0=buf, rot=True)
        assert np.array_equal(c[0][s_], r["o"][0])


# ---------------------------------------------------------------- FP8 (E4M3) window buffer (variant)
def test_round_e4m3_golden():
    """Nearest E4M3 value, ties to even, worked by hand from the format
    (bias 7, 3 mantissa bits, step 2^(e-3) in [2^e, 2^(e+1)), subnormal
    step 2^-9, largest finite 448)."""
    cases = [
        (1.0, 1.0),
        (1.0625, 1.0),                # tie between 1.0 (M=000) and 1.125 (M=001): even -> 1.0
        (1.1875, 1.25),               # tie between 1.125 (001) and 1.25 (010): even -> 1.25
        (1.07, 1.125),                # just above the tie -> up
        (17.0, 16.0),                 # step 2 in [16, 32): 8.5 steps -> 8 (even)
        (19.0, 20.0),                 # 9.5 steps -> 10 (even)
        (447.0, 448.0),               # step 32 in [256, 512): 13.97 -> 14
        (-240.0, -240.0),             # on the grid
        (1.5 * 2.0 ** -9, 2.0 ** -8),  # subnormal tie: 1.5 steps -> 2 (even)
        (0.5 * 2.0 ** -9, 0.0),       # subnormal tie: 0.5 steps -> 0 (even)
        (0.75 * 2.0 ** -9, 2.0 ** -9),
        (2.0 ** -6, 2.0 ** -6),       # smallest normal
        (0.0, 0.0),
    ]
    x = np.array([c[0] for c in cases], F32)
    want = np.array([c[1] for c in cases], F32)
    assert np.array_equal(O.round_e4m3(x), want)


def test_round_e4m3_matches_torch_cast():
    """The same rounding as torch's fp32 -> float8_e4m3fn cast (a library
    routine), over the normal and the subnormal range."""
    import torch
    g = np.random.default_rng(33)
    x = np.concatenate([g.uniform(-448, 448, 20000), g.uniform(-0.03, 0.03, 20000),
                        g.standard_normal(20000) * np.exp(g.uniform(-12, 5, 20000))])
    x = np.clip(x, -448, 448).astype(F32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(O.round_e4m3(x), t)


def test_quantize_e4m3_vector_properties():
    """Per-vector E4M3: the largest entry lands on +-448 * scale; every
    stored value is within half a grid step (times the scale) of its input:
    at most |x| / 16 on the normal range, 2^-10 * scale below it; a zero
    vector stores zeros with scale 0."""
    g = np.random.default_rng(34)
    x = (g.standard_normal((64, 128)) * np.exp(g.uniform(-6, 6, (64, 1)))).astype(F32)
    x[5] = 0.0
    vals, c, s = O.quantize_e4m3_vector(x)
    assert s[5] == 0 and np.all(vals[5] == 0)
    nz = s > 0
    amax_i = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(c[nz, amax_i[nz]]) == 448.0)
    err = np.abs(vals.astype(np.float64) - x)
    q = np.abs(x) / np.where(s > 0, s, 1)[:, None]
    bound = np.where(q >= 2.0 ** -6, np.abs(x) / 16.0, 2.0 ** -10 * s[:, None]) * (1 + 2.0 ** -20)
    assert np.all(err <= bound + 1e-30)
    assert np.array_equal(vals, (c * s[:, None]).astype(F32))


def test_buf_fp8_current_write_exact_and_stored_quantized():
    """With the FP8 buffer the step's own write is used exactly (the output
    equals the fp32 buffer's), the stored slot is the E4M3 vector pair of
    the write, and the next step replays the stored values."""
    W = 8
    d = wl.decode_batch(B=2, H=2, dk=16, dv=16, W=W, seed=9, fill=np.array([1, 3]), poison=False)
    codes, scales = O.quantize_rows(d["state"])
    bk = O.quantize_e4m3_vector(d["buf_k"])[0]
    bv = O.quantize_e4m3_vector(d["buf_v"])[0]
    args = (codes, scales, bk, bv, d["buf_alpha"], d["buf_beta"], d["fill"], W)
    a = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], *args)
    b = O.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], *args, buf_fp8=True)
    assert np.array_equal(a[0], b[0])
    for s_ in range(2):
        f = int(d["fill"][s_])
        assert np.array_equal(b[3][s_, :, f], O.quantize_e4m3_vector(a[3][s_, :, f])[0])
        assert np.array_equal(b[4][s_, :, f], O.quantize_e4m3_vector(a[4][s_, :, f])[0])
        assert not np.array_equal(b[3][s_, :, f], a[3][s_, :, f])
    x = wl.decode_tokens(B=2, H=2, dk=16, dv=16, step=1, seed=10)
    c = O.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], *b[1:7], b[7], W, buf_fp8=True)
    for s_ in range(2):
        f = int(b[7][s_])
        buf = {"k": np.moveaxis(b[3][s_, :, :f], 1, 0), "v": np.moveaxis(b[4][s_, :, :f], 1, 0),
               "alpha": b[5][s_, :, :f].T, "beta": b[6][s_, :, :f].T}
        r = O.run_windowed(x["q"][s_][None], x["k"][s_][None], x["v"][s_][None],
                           x["alpha"][s_][None], x["beta"][s_][None], W=W, codes0=b[1][s_],
                           scale0=b[2][s_], buffer0=buf)
        assert np.array_equal(c[0][s_], r["o"][0])


# ---------------------------------------------------------------- uniform 4-bit state
def test_codec4_golden_rows():
    """The 4-bit codec (scale = absmax / 7, codes = clamp(rne(x / scale),
    -7, 7)) on rows worked by hand: with absmax 7 the scale is 1 and the
    codes are x rounded half to even; with absmax 14 the scale is 2; a zero
    row gets scale 0 (Low-Bit GDN ..., abstract: the "@4" budget; the
    rule is the 8-bit one with 15 levels)."""
    x = np.array([[3.5, -7.0, 1.75, 0.0, 0.25, 2.5, -0.5, 6.5],
                  [14.0, -3.0, 5.0, 1.0, 0.0, -14.0, 13.0, 3.0],
                  [0.0] * 8], F32)
    codes, scale = O.quantize_rows(x, qmax=7)
    assert scale.tolist() == [1.0, 2.0, 0.0]
    assert codes.tolist() == [[4, -7, 2, 0, 0, 2, 0, 6],
                              [7, -2, 2, 0, 0, -7, 6, 2],
                              [0] * 8]


def test_codec4_properties_random():
    """Every code within [-7, 7]; the absmax entry maps to +-7; each entry
    within half a step of code * scale."""
    g = np.random.default_rng(41)
    x = (g.standard_normal((200, 128)) * g.uniform(0.01, 10, (200, 1))).astype(F32)
    codes, scale = O.quantize_rows(x, qmax=7)
    assert np.abs(codes).max() <= 7
    top = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(codes[np.arange(200), top]) == 7)
    err = np.abs(x.astype(F64) - codes.astype(F64) * scale[:, None].astype(F64))
    assert np.all(err <= scale[:, None].astype(F64) * (0.5 + 1e-6))


def test_decode_4bit_calls_equal_one_run():
    """Decode calls with the 4-bit state equal one windowed run with the
    4-bit codec (the same reading as for 8 bits), and every stored code
    stays within [-7, 7]."""
    g = np.random.default_rng(43)
    B, H, d, W, T = 2, 2, 8, 4, 11
    q, k, v, a, b = _rand_tokens(g, T, B * H, d, d)
    r = O.run_windowed(q, k, v, a, b, W=W, qmax=7)
    codes = np.zeros((B, H, d, d), np.int8)
    scales = np.zeros((B, H, d), F32)
    bk = np.full((B, H, W, d), np.nan, F32)
    bv = np.full((B, H, W, d), np.nan, F32)
    ba = np.full((B, H, W), np.nan, F32)
    bb = np.full((B, H, W), np.nan, F32)
    fill = np.zeros(B, np.int32)
    rs = lambda x: x.reshape((B, H) + x.shape[1:])  # noqa: E731
    for t in range(T):
        ot, codes, scales, bk, bv, ba, bb, fill = O.decode_step(
            rs(q[t]), rs(k[t]), rs(v[t]), rs(a[t]), rs(b[t]), codes, scales, bk, bv, ba, bb, fill, W,
            qmax=7)
        assert np.array_equal(ot.reshape(B * H, d), r["o"][t])
        assert np.abs(codes).max() <= 7
    assert np.array_equal(codes.reshape(B * H, d, d), r["codes"])
    assert np.array_equal(scales.reshape(B * H, d), r["scale"])
    # the 4-bit state is coarser: the same run at 8 bits differs
    r8 = O.run_windowed(q, k, v, a, b, W=W)
    assert not np.array_equal(r8["codes"], r["codes"])
