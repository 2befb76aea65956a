"""Plant plausible mistakes in the oracle (CPU only) and check the pins catch them.

Each mutant replaces one oracle function for the duration of one test; the
pins used are the hand-derived worked example and the beta = 1 read-back
property, which do not depend on the oracle being right.
"""

import numpy as np
import pytest

import oracle.gdnq_oracle as G
from conftest import read_golden
from test_oracle_pins import _worked

F32 = np.float32


def _outer(a, b):
    return a[..., :, None] * b[..., None, :]


def _mut_decay_after_erase(S, k, v, a, b):
    Sk = np.matmul(S, k[..., :, None])[..., 0]
    return a[..., None, None] * S - b[..., None, None] * _outer(Sk, k) + b[..., None, None] * _outer(v, k)


def _mut_sign(S, k, v, a, b):
    Sk = np.matmul(S, k[..., :, None])[..., 0]
    return a[..., None, None] * (S + b[..., None, None] * _outer(Sk, k)) + b[..., None, None] * _outer(v, k)


def _mut_no_erase(S, k, v, a, b):
    return a[..., None, None] * S + b[..., None, None] * _outer(v, k)


def _mut_transposed_write(S, k, v, a, b):
    Sk = np.matmul(S, k[..., :, None])[..., 0]
    return a[..., None, None] * (S - b[..., None, None] * _outer(Sk, k)) + b[..., None, None] * _outer(k, v)


def _mut_decayed_write(S, k, v, a, b):
    Sk = np.matmul(S, k[..., :, None])[..., 0]
    return a[..., None, None] * (S - b[..., None, None] * _outer(Sk, k) + b[..., None, None] * _outer(v, k))


def _mut_erase_with_q_side(S, k, v, a, b):  # erase uses S^T k
    Sk = np.matmul(np.swapaxes(S, -1, -2), v[..., :, None] * 0 + k[..., :, None])[..., 0]
    return a[..., None, None] * (S - b[..., None, None] * _outer(Sk, k)) + b[..., None, None] * _outer(v, k)


def _worked_example_holds():
    W, q, k, v, a, b, o, c2, s2, cf, sf = _worked()
    try:
        r = G.run_windowed(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None], W=W)
    except Exception:
        return False
    return (np.array_equal(r["o"][:, 0], o.astype(F32)) and np.array_equal(r["codes"][0], cf)
            and np.array_equal(r["scale"][0], sf))


def _readback_holds():
    g = np.random.default_rng(0)
    T, N, d = 7, 2, 8
    k = g.standard_normal((T, N, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((T, N, d))
    a = g.uniform(0.9, 0.99, (T, N))
    b = np.ones((T, N))
    S0 = g.standard_normal((N, d, d)).astype(F32)
    codes, scale = G.quantize_rows(S0)
    r = G.run_windowed(k, k, v, a, b, W=3, codes0=codes, scale0=scale, dtype=np.float64)
    return np.max(np.abs(r["o"] - v)) < 1e-9


@pytest.mark.parametrize("mutant", [_mut_decay_after_erase, _mut_sign, _mut_no_erase,
                                    _mut_transposed_write, _mut_decayed_write,
                                    _mut_erase_with_q_side])
def test_step_mutant_is_caught(monkeypatch, mutant):
    assert _worked_example_holds() and _readback_holds()
    monkeypatch.setattr(G, "gdn_step", mutant)
    assert not (_worked_example_holds() and _readback_holds())


def _codec_golden_holds():
    g = read_golden("codec_rows.txt")
    for row, sc, cd in zip(g["row"], g["scale"], g["codes"]):
        x = np.array([float(v) for v in row.split()], F32)[None]
        codes, scale = G.quantize_rows(x)
        if scale[0] != F32(float(sc)) or codes[0].tolist() != [int(v) for v in cd.split()]:
            return False
    return True


def _codec_half_away(x):
    x32 = np.asarray(x, F32)
    s = (np.max(np.abs(x32), -1) / F32(127)).astype(F32)
    d = np.where(s > 0, s, F32(1))
    r = x32 / d[..., None]
    c = np.sign(r) * np.floor(np.abs(r) + 0.5)
    return np.clip(c, -127, 127).astype(np.int8), s


def _codec_128(x):
    x32 = np.asarray(x, F32)
    s = (np.max(np.abs(x32), -1) / F32(128)).astype(F32)
    d = np.where(s > 0, s, F32(1))
    return np.clip(np.rint(x32 / d[..., None]), -127, 127).astype(np.int8), s


def _codec_no_abs(x):
    x32 = np.asarray(x, F32)
    s = (np.max(x32, -1) / F32(127)).astype(F32)
    d = np.where(s > 0, s, F32(1))
    return np.clip(np.rint(x32 / d[..., None]), -127, 127).astype(np.int8), s


@pytest.mark.parametrize("mutant", [_codec_half_away, _codec_128, _codec_no_abs])
def test_codec_mutant_is_caught(monkeypatch, mutant):
    assert _codec_golden_holds()
    monkeypatch.setattr(G, "quantize_rows", mutant)
    assert not _codec_golden_holds()


def test_window_off_by_one_is_caught(monkeypatch):
    """A window that closes one token late changes the worked example."""
    W, q, k, v, a, b, o, c2, s2, cf, sf = _worked()
    r = G.run_windowed(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None], W=W + 1)
    assert not np.array_equal(r["o"][:, 0], o.astype(F32))


# ---------------------------------------------------------------- bf16 buffer rounding
def _mut_round_truncate(x):  # drop the low bits (round toward zero)
    u = np.ascontiguousarray(np.asarray(x, dtype=F32)).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(F32)


def _mut_round_half_up(x):  # ties away from zero instead of to even
    u = np.ascontiguousarray(np.asarray(x, dtype=F32)).view(np.uint32).astype(np.uint64)
    return (((u + 0x8000) & 0xFFFF0000).astype(np.uint32)).view(F32)


@pytest.mark.parametrize("mut", [_mut_round_truncate, _mut_round_half_up])
def test_bf16_rounding_mutants_are_caught(mut, monkeypatch):
    import test_oracle_pins as P
    monkeypatch.setattr(G, "round_bf16", mut)
    monkeypatch.setattr(P.O, "round_bf16", mut)
    with pytest.raises(AssertionError):
        P.test_round_bf16_golden()


# ---------------------------------------------------------------- E4M3 buffer rounding
def _mut_e4m3_truncate(x):  # round toward zero on the E4M3 grid
    x = np.asarray(x, dtype=F32).astype(np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(ex.astype(np.int64) - 1, -6) - 3)
    return (np.sign(x) * np.minimum(np.floor(a / step) * step, 448.0)).astype(F32)


def _mut_e4m3_half_up(x):  # ties away from zero
    x = np.asarray(x, dtype=F32).astype(np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(ex.astype(np.int64) - 1, -6) - 3)
    return (np.sign(x) * np.minimum(np.floor(a / step + 0.5) * step, 448.0)).astype(F32)


def _mut_e4m3_no_subnormals(x):  # flush the subnormal range to zero
    r = G.__dict__["_round_e4m3_ref"](x)
    return np.where(np.abs(r) < 2.0 ** -6, F32(0), r).astype(F32)


@pytest.mark.parametrize("mut", [_mut_e4m3_truncate, _mut_e4m3_half_up, _mut_e4m3_no_subnormals])
def test_e4m3_rounding_mutants_are_caught(mut, monkeypatch):
    import test_oracle_pins as P
    monkeypatch.setitem(G.__dict__, "_round_e4m3_ref", G.round_e4m3)
    monkeypatch.setattr(G, "round_e4m3", mut)
    monkeypatch.setattr(P.O, "round_e4m3", mut)
    with pytest.raises(AssertionError):
        P.test_round_e4m3_golden()
