"""Pins of the oracle's Pure-Write sliding window ("Low-Bit GDN Recurrent-State
Quantization ...", abstract: pure writes kept apart, propagated through the
full GDN transition, merged into the low-bit historical state when they leave
the window).  Each test names the mistake it would catch; none re-types the
oracle's own formula."""

import numpy as np
import pytest

import oracle as O
import workloads as wl
from conftest import read_golden

F32, F64 = np.float32, np.float64


def _rows(s):
    return np.array([[float(x) for x in r.split()] for r in s.split("|")])


def _golden():
    g = read_golden("sliding_worked_example.txt")
    k = _rows(g["k"][0])
    return dict(q=_rows(g["q"][0]), k=k, v=_rows(g["v"][0]),
                alpha=np.array([float(x) for x in g["alpha"][0].split()]),
                beta=np.array([float(x) for x in g["beta"][0].split()]),
                o=_rows(g["o"][0]), codes=_rows(g["codes"][0]).reshape(-1, 2, 2),
                scale=_rows(g["scale"][0]), W=int(g["W"][0]))


@pytest.mark.parametrize("dtype", [F32, F64])
def test_sliding_worked_example_exact(dtype):
    """The hand-derived example (tests/golden/sliding_worked_example.txt),
    one decode call per token through the ring buffer: outputs, and the
    historical codes and scales after every token, exactly.  Catches a window
    key that is not propagated (t2), propagation without the erase term (t3),
    a window one write too long (t2), an output taken after the
    requantization (t3), a historical state that skips the transition (t3),
    and a round-half-away codec (t3's 63.5)."""
    g = _golden()
    W = g["W"]
    codes = np.zeros((1, 1, 2, 2), np.int8)
    scales = np.zeros((1, 1, 2), F32)
    bk = np.full((1, 1, W, 2), np.nan, F32)
    bv = np.full((1, 1, W, 2), np.nan, F32)
    ba = np.full((1, 1, W), np.nan, F32)
    bb = np.full((1, 1, W), np.nan, F32)
    fill = np.zeros(1, np.int32)
    for t in range(4):
        x = [np.asarray(g[n][t], dtype)[None, None] for n in ("q", "k", "v")]
        ab = [np.asarray([[g[n][t]]], dtype) for n in ("alpha", "beta")]
        o, codes, scales, bk, bv, ba, bb, fill = O.decode_step_sliding(*x, *ab, codes, scales, bk, bv, ba, bb,
                                                                       fill, W, dtype=dtype)
        assert o[0, 0].tolist() == g["o"][t].tolist(), t
        assert codes[0, 0].tolist() == g["codes"][t].tolist(), t
        exp = [F32(float(s)) for s in g["scale"][t]]
        assert scales[0, 0].tolist() == exp, t


def test_sliding_no_window_is_tumbling_window_of_one():
    """W = 0 (every write merges at once) is the tumbling window of one token
    (requantize after every token), bitwise: the two readings coincide there."""
    x = wl.gdn_prefill(B=1, T=40, H=3, dk=32, dv=16, seed=3)
    tn = lambda a: np.ascontiguousarray(a[0])  # [T, H, ...]
    g = np.random.default_rng(4)
    S0 = (g.standard_normal((3, 16, 32)) * 0.5).astype(F32)
    c0, s0 = O.quantize_rows(S0)
    a = O.run_sliding(tn(x["q"]), tn(x["k"]), tn(x["v"]), tn(x["alpha"]), tn(x["beta"]), W=0, codes0=c0, scale0=s0)
    b = O.run_windowed(tn(x["q"]), tn(x["k"]), tn(x["v"]), tn(x["alpha"]), tn(x["beta"]), W=1, codes0=c0, scale0=s0)
    assert np.array_equal(a["o"], b["o"])
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scale"], b["scale"])


@pytest.mark.parametrize("W", [None, 50])
def test_sliding_never_merging_is_the_unquantized_recurrence(W):
    """From a zero state with a window no write leaves (W >= T, or None), the
    historical part stays 0 and the state is the exact recurrence: equal to
    the unquantized token-by-token run within fp64 rounding."""
    x = wl.gdn_prefill(B=1, T=40, H=2, dk=16, dv=8, seed=5)
    tn = lambda a: np.ascontiguousarray(a[0])
    a = O.run_sliding(tn(x["q"]), tn(x["k"]), tn(x["v"]), tn(x["alpha"]), tn(x["beta"]), W=W, dtype=F64)
    b = O.run_windowed(tn(x["q"]), tn(x["k"]), tn(x["v"]), tn(x["alpha"]), tn(x["beta"]), W=None, dtype=F64)
    assert not a["codes"].any() and not a["scale"].any()
    assert np.max(np.abs(a["o"] - b["o"])) <= 1e-12 * np.max(np.abs(b["o"]))


def _dense_A(k, a, b):
    d = len(k)
    return a * (np.eye(d) - b * np.outer(k, k))


def test_sliding_one_token_is_one_full_step_of_the_dequantized_state():
    """Brute force with dense transition matrices, fp64: rebuild the full
    state before a token from the stored historical codes and the raw window
    (each write times the product of the dense transitions after it), apply
    one full gated delta-rule step, and compare with the state the oracle
    forms (historical part before requantization plus its propagated
    window), at every token of a run with merges.  Catches a merge with an
    unpropagated key, a missing or misplaced transition, and a write merged
    twice or never."""
    T, dk, dv, W = 14, 8, 5, 3
    g = np.random.default_rng(6)
    q = g.standard_normal((T, 1, dk))
    k = g.standard_normal((T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((T, 1, dv))
    al = g.uniform(0.5, 1.0, (T, 1))
    be = g.uniform(0.0, 1.0, (T, 1))
    c0, s0 = O.quantize_rows(g.standard_normal((1, dv, dk)).astype(F32))
    codes, scale, win = c0, s0, None
    for t in range(T):
        # the full state before token t, from the stored parts, by dense products
        S = O.dequantize(codes, scale, F64)[0]
        n = 0 if win is None else len(win["k"])
        for i in range(n):
            P = np.eye(dk)
            for j in range(i + 1, n):
                P = P @ _dense_A(win["k"][j][0], win["alpha"][j][0], win["beta"][j][0])
            S = S + win["beta"][i][0] * np.outer(win["v"][i][0], win["k"][i][0]) @ P
        S_ref = S @ _dense_A(k[t, 0], al[t, 0], be[t, 0]) + be[t, 0] * np.outer(v[t, 0], k[t, 0])
        r = O.run_sliding(q[t:t + 1], k[t:t + 1], v[t:t + 1], al[t:t + 1], be[t:t + 1], W=W, codes0=codes,
                          scale0=scale, window0=win, dtype=F64)
        assert np.max(np.abs(r["S"][0] - S_ref)) <= 1e-12 * np.max(np.abs(S_ref)), t
        assert np.allclose(r["o"][0, 0], S_ref @ q[t, 0], rtol=1e-12, atol=1e-12)
        assert r["n"] == min(n + 1, W)
        codes, scale, win = r["codes"], r["scale"], r["window"]


def test_sliding_decode_calls_equal_one_run():
    """T decode calls through the ring buffer (fills walking past W and
    wrapping) equal one run of T tokens, bitwise, and the ring's raw writes
    are the window's, in order.  Catches ring-order and slot mistakes."""
    B, H, dk, dv, W, T = 2, 2, 16, 8, 5, 17
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=dk, dv=dv, seed=7)
    g = np.random.default_rng(8)
    c0, s0 = O.quantize_rows((g.standard_normal((B, H, dv, dk)) * 0.5).astype(F32))
    ref = [O.run_sliding(x["q"][b], x["k"][b], x["v"][b], x["alpha"][b], x["beta"][b], W=W, codes0=c0[b],
                         scale0=s0[b]) for b in range(B)]
    codes, scales = c0, s0
    bk = np.full((B, H, W, dk), np.nan, F32)
    bv = np.full((B, H, W, dv), np.nan, F32)
    ba = np.full((B, H, W), np.nan, F32)
    bb = np.full((B, H, W), np.nan, F32)
    fill = np.zeros(B, np.int32)
    for t in range(T):
        o, codes, scales, bk, bv, ba, bb, fill = O.decode_step_sliding(
            x["q"][:, t], x["k"][:, t], x["v"][:, t], x["alpha"][:, t], x["beta"][:, t], codes, scales,
            bk, bv, ba, bb, fill, W)
        for b in range(B):
            assert np.array_equal(o[b], ref[b]["o"][t]), (t, b)
    for b in range(B):
        assert np.array_equal(codes[b], ref[b]["codes"]) and np.array_equal(scales[b], ref[b]["scale"])
        slots, _, _ = O.sliding_ring_slots(fill[b], W)
        assert np.array_equal(bk[b][:, slots].transpose(1, 0, 2), ref[b]["window"]["k"])
    assert fill.tolist() == [W + T % W] * B


def test_sliding_ring_slots():
    """The ring's bookkeeping, by hand: W = 3."""
    assert O.sliding_ring_slots(0, 3) == ([], 0, 1)
    assert O.sliding_ring_slots(2, 3) == ([0, 1], 2, 3)
    assert O.sliding_ring_slots(3, 3) == ([0, 1, 2], 0, 4)
    assert O.sliding_ring_slots(4, 3) == ([1, 2, 0], 1, 5)
    assert O.sliding_ring_slots(5, 3) == ([2, 0, 1], 2, 3)
    assert O.sliding_ring_slots(1, 1) == ([0], 0, 1)


def test_sliding_identity_transition_keeps_state():
    """alpha = 1, beta = 0: nothing is written or erased; the output is the
    stored state times q at every token and the codes never change (the
    requantization is idempotent on a dequantized state; scales within one
    ulp)."""
    T, H, d, W = 12, 3, 16, 4
    g = np.random.default_rng(9)
    c0, s0 = O.quantize_rows((g.standard_normal((H, d, d)) * 0.5).astype(F32))
    q = g.standard_normal((T, H, d)).astype(F32)
    k = g.standard_normal((T, H, d)).astype(F32)
    r = O.run_sliding(q, k, g.standard_normal((T, H, d)).astype(F32), np.ones((T, H), F32),
                      np.zeros((T, H), F32), W=W, codes0=c0, scale0=s0)
    S = O.dequantize(c0, s0, F32)
    for t in range(T):
        assert np.allclose(r["o"][t], np.matmul(S, q[t][..., None])[..., 0], rtol=1e-6, atol=1e-6)
    assert np.array_equal(r["codes"], c0)
    assert np.all(np.abs(r["scale"] - s0) <= np.spacing(s0))


# ---------------------------------------------------------------- mutants
def _key_not_propagated(x, k, a, b):
    return x


def _key_decay_only(x, k, a, b):
    return a[..., None] * x


def _key_sign_flipped(x, k, a, b):
    return a[..., None] * (x + b[..., None] * np.sum(k * x, axis=-1)[..., None] * k)


def _history_skips_transition(X, k, a, b):
    return X


@pytest.mark.parametrize("name,target,mutant", [
    ("window key not propagated", "propagate_key", _key_not_propagated),
    ("propagation without the erase", "propagate_key", _key_decay_only),
    ("erase with the wrong sign", "propagate_key", _key_sign_flipped),
    ("historical state skips the transition", "gdn_transition", _history_skips_transition),
])
def test_sliding_pins_catch_mutants(name, target, mutant, monkeypatch):
    """Each planted mistake makes the worked example or the dense-product pin fail."""
    import oracle.gdnq_oracle as G
    monkeypatch.setattr(G, target, mutant)
    caught = 0
    for pin in (lambda: test_sliding_worked_example_exact(F64),
                test_sliding_one_token_is_one_full_step_of_the_dequantized_state):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, name
