"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything.

Pointers here are fake addresses that the host code compares but never
dereferences; every call below fails validation, so no kernel is launched.
"""

import os
import re

import pytest

from quantized_recurrent_state_gdnq_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib


def _declared():
    txt = open(os.path.join(ROOT, "include", "gdnq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gdnq_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert L.gdnq_version() >= 100
    for s in range(9):
        assert L.gdnq_status_string(s)


def test_sync_debug_mode_read_at_load():
    """GDNQ_SYNC_DEBUG=1 at load switches every call to synchronize its
    stream; any other value, or none, leaves the library asynchronous."""
    import subprocess
    import sys
    code = "from quantized_recurrent_state_gdnq_amd import _lib; print(_lib.lib.gdnq_sync_debug())"
    for val, want in (("1", "1"), ("0", "0"), ("yes", "0"), (None, "0")):
        env = {k: v for k, v in os.environ.items() if k != "GDNQ_SYNC_DEBUG"}
        if val is not None:
            env["GDNQ_SYNC_DEBUG"] = val
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        assert r.stdout.strip() == want, (val, r.stdout)


class Fake:
    """Distinct, 16-byte-aligned, never-dereferenced addresses."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes=1 << 24):
        p = self.next
        self.next += ((nbytes + (1 << 20)) // (1 << 20) + 1) << 20
        return p


def _decode_args(fake, B=2, H=2, d=128, W=8):
    return dict(q=fake(), k=fake(), v=fake(), alpha=fake(), beta=fake(), codes=fake(),
                scales=fake(), buf_k=fake(), buf_v=fake(), buf_alpha=fake(), buf_beta=fake(),
                fill_in=fake(), fill_out=fake(), o=fake())


def _decode(params, a, stream=None):
    return _lib.decode_step(params, a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["codes"],
                            a["scales"], a["buf_k"], a["buf_v"], a["buf_alpha"], a["buf_beta"],
                            a["fill_in"], a["fill_out"], a["o"], stream)


def _p(B=2, H=2, dk=128, dv=128, W=8, ind=1, outd=1, flags=0):
    return _lib.DecodeParams(B, H, dk, dv, W, ind, outd, flags)


@pytest.mark.parametrize("params,status", [
    (_p(dk=96), 2), (_p(dv=32), 2), (_p(B=1025), 2), (_p(W=0), 2), (_p(W=65), 2), (_p(H=0), 2), (_p(B=-1), 2),
    (_p(ind=2), 3), (_p(outd=5), 3), (_p(flags=2), 8), (_p(flags=4), 8), (_p(flags=512), 8),
    (_p(flags=16 | 2), 8), (_p(flags=16 | 32), 8),
    (_p(flags=128 | 16), 8), (_p(flags=128 | 32), 8), (_p(flags=128 | 64), 8), (_p(flags=256), 8),
])
def test_decode_rejects_bad_params(params, status):
    a = _decode_args(Fake())
    assert _decode(params, a) == status
    assert L.gdnq_last_error()


def test_decode_null_params_and_pointers():
    assert L.gdnq_decode_step(None, *([None] * 15)) == 1
    for name in ["q", "codes", "buf_beta", "fill_in", "fill_out", "o"]:
        a = _decode_args(Fake())
        a[name] = None
        assert _decode(_p(), a) == 1, name
        assert name.encode() in L.gdnq_last_error()


def test_decode_misaligned():
    a = _decode_args(Fake())
    a["buf_v"] += 4
    assert _decode(_p(), a) == 4
    assert b"buf_v" in L.gdnq_last_error()


def test_decode_aliasing():
    a = _decode_args(Fake())
    a["fill_out"] = a["fill_in"]
    assert _decode(_p(), a) == 5
    a = _decode_args(Fake())
    a["o"] = a["q"]
    assert _decode(_p(), a) == 5
    a = _decode_args(Fake())
    a["buf_v"] = a["buf_k"] + 256  # partial overlap
    assert _decode(_p(), a) == 5


def test_decode_bf16_buffer_spans():
    """Under GDNQ_FLAG_BUF_BF16 the window buffers hold 2-byte entries: a
    buf_v placed right after a bf16-sized buf_k is disjoint from it (the
    only overlap reported is a planted one between o and fill_out, checked
    later), while the same placement overlaps an fp32-sized buf_k."""
    B, H, d, W = 2, 2, 128, 8
    a = _decode_args(Fake())
    a["buf_v"] = a["buf_k"] + B * H * W * d * 2
    a["o"] = a["fill_out"]
    assert _decode(_p(flags=16), a) == 5
    err = L.gdnq_last_error()
    assert b"buf" not in err and b"fill_out overlaps o" in err, err
    a = _decode_args(Fake())
    a["buf_v"] = a["buf_k"] + B * H * W * d * 2 - 16
    assert _decode(_p(flags=16), a) == 5
    assert b"buf_k overlaps buf_v" in L.gdnq_last_error()
    a = _decode_args(Fake())
    a["buf_v"] = a["buf_k"] + B * H * W * d * 2
    assert _decode(_p(flags=0), a) == 5
    assert b"buf_k overlaps buf_v" in L.gdnq_last_error()


def test_decode_fp8_buffer_spans():
    """Under GDNQ_FLAG_BUF_FP8 each window buffer holds one byte per entry
    followed by one fp32 scale per vector: a buf_v placed right after
    B*H*W*(d + 4) bytes of buf_k is disjoint from it, 16 bytes earlier it
    overlaps the scales."""
    B, H, d, W = 2, 2, 128, 8
    a = _decode_args(Fake())
    a["buf_v"] = a["buf_k"] + B * H * W * (d + 4)
    a["o"] = a["fill_out"]
    assert _decode(_p(flags=32), a) == 5
    err = L.gdnq_last_error()
    assert b"buf" not in err and b"fill_out overlaps o" in err, err
    a = _decode_args(Fake())
    a["buf_v"] = a["buf_k"] + B * H * W * (d + 4) - 16
    assert _decode(_p(flags=32), a) == 5
    assert b"buf_k overlaps buf_v" in L.gdnq_last_error()


def test_decode_empty_batch_is_noop():
    a = {k: None for k in _decode_args(Fake())}
    assert _decode(_p(B=0), a) == 0


def _pp(B=1, T=128, H=2, dk=128, dv=128, C=64, W=64, ind=1, outd=1, flags=0):
    return _lib.PrefillParams(B, T, H, dk, dv, C, W, ind, outd, flags)


def _prefill(params, fake, **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), beta=fake(), init_codes=None,
             init_scales=None, o=fake(), codes=fake(), scales=fake(), state_f32=None,
             workspace=None, ws=0, buf_k=None, buf_v=None, buf_alpha=None, buf_beta=None, fill_out=None)
    a.update(over)
    return _lib.prefill_chunked(params, a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                a["init_codes"], a["init_scales"], a["o"], a["codes"],
                                a["scales"], a["state_f32"], a["workspace"], a["ws"], None,
                                buf_k=a["buf_k"], buf_v=a["buf_v"], buf_alpha=a["buf_alpha"],
                                buf_beta=a["buf_beta"], fill_out=a["fill_out"])


@pytest.mark.parametrize("params,status", [
    (_pp(C=8, W=8), 2), (_pp(T=100), 1), (_pp(dk=64, dv=128), 2), (_pp(W=0), 2), (_pp(W=-64), 2),
    (_pp(T=48, W=32, C=32), 1),           # not a whole number of windows: the window buffer is required
    (_pp(T=128, W=256), 2),                # likewise, and decode's window is at most 64
    (_pp(T=0, W=(1 << 24) + 64), 2),       # longer than GDNQ_MAX_WINDOW
    (_pp(dk=64, dv=64, flags=1), 8),       # no rotation at d = 64
    (_pp(ind=0), 3), (_pp(outd=3), 3), (_pp(flags=4), 8), (_pp(flags=16), 8),
    (_pp(flags=32), 8),
    (_pp(flags=8), 2),                     # no requantization: codes and scales must be NULL
    (_pp(dv=64, flags=2 | 4 | 8), 8),      # not for SSD
])
def test_prefill_rejects_bad_params(params, status):
    assert _prefill(params, Fake()) == status


def test_prefill_gdn_rotation_flag():
    """GDNQ_FLAG_WHT is accepted by every GDN prefill call (a larger workspace:
    the rotated q and k)."""
    p0, p1 = _pp(), _pp(flags=1)
    assert L.gdnq_prefill_workspace_size(p1) == L.gdnq_prefill_workspace_size(p0) + 2 * 1 * 128 * 2 * 128 * 2
    f = Fake()
    assert _prefill(p1, f, ws=L.gdnq_prefill_workspace_size(p0), workspace=f()) == 6  # too small
    assert L.gdnq_prefill_handoff_workspace_size(p1) == L.gdnq_prefill_handoff_workspace_size(p0) + 2 * 128 * 2 * 128 * 2
    assert L.gdnq_prefill_varlen_workspace_size(p1) == L.gdnq_prefill_varlen_workspace_size(p0) + 2 * 128 * 2 * 128 * 2


def test_prefill_gdn_contract():
    f = Fake()
    assert _prefill(_pp(), f, beta=None) == 1
    assert _prefill(_pp(), f, state_f32=f()) == 2
    c = f()
    assert _prefill(_pp(), f, init_codes=c) == 1           # init_scales missing
    assert _prefill(_pp(), f, o=None) == 1
    q = f()
    assert _prefill(_pp(), f, q=q, o=q) == 5               # output over an input


def test_prefill_ssd_contract():
    f = Fake()
    ssd = _pp(dv=64, flags=2 | 1 | 4)
    assert _prefill(ssd, f, beta=None, codes=None, scales=None) == 1          # state_f32 missing
    assert _prefill(ssd, f, codes=None, scales=None, state_f32=f()) == 2      # beta given
    # d_k = 64 runs on operand rows widened to 128 and a padded state: a
    # workspace even for plain bf16 operands
    assert _prefill(_pp(dk=64, dv=64, flags=2), f, beta=None, codes=None, scales=None,
                    state_f32=f()) == 6
    assert _prefill(_pp(dk=96, dv=64, flags=2), f, beta=None, codes=None, scales=None,
                    state_f32=f()) == 2


def test_ssd_workspace_by_flags():
    """SSD workspace: none for plain bf16 operands, the rotated bf16 rows with
    the rotation alone, the int8 codes and scales with int8 operands; at
    d_k = 64 the widened operand rows and a padded fp32 state."""
    rows = 1 * 128 * 2
    assert L.gdnq_prefill_workspace_size(_pp(dv=64, flags=2)) == 0
    assert L.gdnq_prefill_workspace_size(_pp(dv=64, flags=2 | 1)) == 2 * rows * 128 * 2
    assert L.gdnq_prefill_workspace_size(_pp(dv=64, flags=2 | 4)) == 2 * rows * 128 + 2 * rows * 4
    assert L.gdnq_prefill_workspace_size(_pp(dv=64, flags=2 | 1 | 4)) == 2 * rows * 128 + 2 * rows * 4
    # d_k = 64: operand rows widened to 128 (bf16 even with neither flag), then
    # at a 256-byte boundary the state [B,H,d_v,128] in fp32
    pad = lambda n: (n + 255) // 256 * 256
    st = 1 * 2 * 64 * 128 * 4
    assert L.gdnq_prefill_workspace_size(_pp(dk=64, dv=64, flags=2)) == pad(2 * rows * 128 * 2) + st
    assert L.gdnq_prefill_workspace_size(_pp(dk=64, dv=64, flags=2 | 1)) == pad(2 * rows * 128 * 2) + st
    assert L.gdnq_prefill_workspace_size(_pp(dk=64, dv=64, flags=2 | 4)) == pad(2 * rows * 128 + 2 * rows * 4) + st
    assert (L.gdnq_prefill_workspace_size(_pp(T=64, H=3, dk=64, dv=128, flags=2 | 1 | 4))
            == pad(2 * 192 * 128 + 2 * 192 * 4) + 3 * 128 * 128 * 4)


def test_window_and_chunk_sizes():
    """GDN prefill takes windows and chunks of 16, 32 or 64.  A window
    below 64 runs on padded copies (a larger workspace, growing as the window
    shrinks); the chunk is a blocking hint that does not change the
    workspace.  The hand-over calls take decode's windows; SSD takes 64."""
    sz = {(W, C): L.gdnq_prefill_workspace_size(_pp(T=256, W=W, C=C)) for W in (16, 32, 64) for C in (16, 32, 64)}
    assert all(v > 0 for v in sz.values())
    for W in (16, 32, 64):
        assert sz[(W, 16)] == sz[(W, 32)] == sz[(W, 64)]
    assert sz[(16, 64)] > sz[(32, 64)] > sz[(64, 64)]
    assert L.gdnq_prefill_workspace_size(_pp(T=48, W=16, C=16)) > 0
    assert L.gdnq_prefill_varlen_workspace_size(_pp(T=256, W=32, C=32)) > 0
    assert L.gdnq_prefill_varlen_workspace_size(_pp(T=256, W=128)) == 0  # decode's windows: 1 .. 64
    assert L.gdnq_prefill_workspace_size(_pp(T=256, dv=64, flags=2 | 4)) > 0
    assert L.gdnq_prefill_workspace_size(_pp(T=256, dv=64, C=32, W=32, flags=2 | 4)) == 0  # SSD: chunk 64


def test_long_windows():
    """Any window: a multiple of 64 runs unpadded (the same workspace as
    W = 64); any other window is padded to whole 64-position chunks (W = 80
    -> 128 positions per window, W = 1 -> 64); the hand-over, varlen and
    resume calls keep decode's 64."""
    base = L.gdnq_prefill_workspace_size(_pp(T=512))
    for W in (128, 256, 512):
        assert L.gdnq_prefill_workspace_size(_pp(T=512, W=W)) == base
    # 160 tokens as two windows of 128 positions: the 256-position run plus its padded copies
    assert L.gdnq_prefill_workspace_size(_pp(T=160, W=80, C=16)) > L.gdnq_prefill_workspace_size(_pp(T=256, W=128))
    # two windows of 48 and one of 96 both run as 128 positions
    assert L.gdnq_prefill_workspace_size(_pp(T=96, W=48, C=16)) == L.gdnq_prefill_workspace_size(_pp(T=96, W=96, C=32))
    # four windows of one token and four of 16 both run as 256 padded positions
    assert L.gdnq_prefill_workspace_size(_pp(T=4, W=1, C=16)) == L.gdnq_prefill_workspace_size(_pp(T=64, W=16, C=16))
    assert L.gdnq_prefill_workspace_size(_pp(T=256, W=1 << 24)) == 0  # T not a multiple of W
    assert L.gdnq_prefill_handoff_workspace_size(_pp(T=256, W=128)) == 0


def test_no_requant_contract():
    """GDNQ_FLAG_NO_REQUANT (gdnq_prefill_chunked, GDN): the final fp32 state
    goes to state_f32; codes and scales must be NULL; any T (no windows)."""
    f = Fake()
    p = _pp(flags=8)
    assert _prefill(p, f, codes=None, scales=None) == 1                      # state_f32 missing
    assert _prefill(p, f, scales=None, state_f32=f()) == 2                   # codes given
    sf = f()
    assert _prefill(p, f, codes=None, scales=None, state_f32=sf, init_codes=sf, init_scales=f()) == 5
    assert L.gdnq_prefill_workspace_size(_pp(T=48, C=16, W=64, flags=8)) > 0  # padded to 64 positions
    assert L.gdnq_prefill_workspace_size(_pp(T=40, C=16, W=64, flags=8)) > 0
    assert L.gdnq_prefill_workspace_size(_pp(T=512, W=64, flags=8)) == L.gdnq_prefill_workspace_size(_pp(T=512))
    assert L.gdnq_prefill_handoff_workspace_size(_pp(flags=8)) == 0
    assert L.gdnq_prefill_varlen_workspace_size(_pp(flags=8)) == 0


def test_workspace_size_is_queryable():
    assert L.gdnq_prefill_workspace_size(None) == 0
    p = _pp()
    assert _lib.prefill_workspace_size(p) >= 0


def test_workspace_sizes():
    """GDN: per chunk-head, T's ten lower 16x16 tiles as three bf16 parts
    (15 KiB) and g (256 B);
    SSD int8: codes and scales of q and k per token row; plain SSD: none."""
    B, T, H = 2, 256, 3
    nch = B * (T // 64) * H
    assert _lib.prefill_workspace_size(_pp(B=B, T=T, H=H)) == nch * (3 * 10 * 256 * 2 + 64 * 4)
    rows = B * T * H
    assert _lib.prefill_workspace_size(_pp(B=B, T=T, H=H, dv=64, flags=2 | 4 | 1)) == rows * (2 * 128 + 8)
    assert _lib.prefill_workspace_size(_pp(B=B, T=T, H=H, dv=64, flags=2)) == 0


def test_quantize_validation():
    f = Fake()
    assert L.gdnq_quantize_state(f(), 0, 128, f(), f(), 0, None) == 0     # empty is a no-op
    assert L.gdnq_quantize_state(f(), 4, 96, f(), f(), 0, None) == 2
    assert L.gdnq_quantize_state(f(), -1, 128, f(), f(), 0, None) == 2
    assert L.gdnq_quantize_state(f(), 4, 128, f(), f(), 2, None) == 8
    assert L.gdnq_quantize_state(None, 4, 128, f(), f(), 0, None) == 1
    assert L.gdnq_quantize_state(f() + 8, 4, 128, f(), f(), 0, None) == 4
    s = f()
    assert L.gdnq_quantize_state(s, 4, 128, s, f(), 0, None) == 5
    # the 4-bit state flag is accepted (the call goes on to the alignment check), alone or with WHT
    assert L.gdnq_quantize_state(f(), 4, 128, f(), f() + 8, 64, None) == 4
    assert L.gdnq_quantize_state(f(), 4, 128, f(), f() + 8, 64 | 1, None) == 4
    assert L.gdnq_quantize_state(f(), 4, 128, f(), f(), 64 | 2, None) == 8


# ---------------------------------------------------------------- prefill hand-over to decode
def _handoff(params, fake, **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), beta=fake(), init_codes=None,
             init_scales=None, o=fake(), codes=fake(), scales=fake(), buf_k=fake(), buf_v=fake(),
             buf_alpha=fake(), buf_beta=fake(), fill_out=fake(), workspace=None, ws=0)
    a.update(over)
    return _lib.prefill_handoff(params, a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                a["init_codes"], a["init_scales"], a["o"], a["codes"], a["scales"],
                                a["buf_k"], a["buf_v"], a["buf_alpha"], a["buf_beta"],
                                a["fill_out"], a["workspace"], a["ws"], None)


@pytest.mark.parametrize("params,status", [
    (_pp(W=128), 2), (_pp(W=0), 2), (_pp(C=8), 2), (_pp(ind=0), 3),  # decode's windows: 1 .. 64
    (_pp(dv=64, flags=2 | 1 | 4), 8),                      # GDN only
    (_pp(dk=64, dv=64, flags=1), 8),                       # no rotation at d = 64
    (_pp(flags=8), 8),                                     # the hand-over requantizes
    (_pp(T=1 << 20, H=8192), 2),                           # one sequence's outputs past 4 GiB
    (_pp(flags=16 | 32), 8),                               # one window-buffer format
])
def test_handoff_rejects_bad_params(params, status):
    assert _handoff(params, Fake()) == status


def test_handoff_windows_and_shapes():
    """Every hand-over call takes decode's windows 1 .. 64, d = 64 and the
    rotation: a window below 64 or d = 64 runs on padded copies (a larger
    workspace); T need not be a multiple of the window."""
    base = _lib.prefill_handoff_workspace_size(_pp(T=100))
    assert base > 0
    for W, C in ((1, 16), (16, 16), (32, 64), (48, 16), (64, 32)):
        assert _lib.prefill_handoff_workspace_size(_pp(T=100, W=W, C=C)) > 0, (W, C)
    assert _lib.prefill_handoff_workspace_size(_pp(T=100, W=16)) > base
    assert _lib.prefill_handoff_workspace_size(_pp(T=100, dk=64, dv=64)) > 0
    assert _lib.prefill_handoff_workspace_size(_pp(T=100, flags=1)) == base + 2 * 100 * 2 * 128 * 2
    assert _lib.prefill_varlen_workspace_size(_pp(T=100, W=32)) > _lib.prefill_varlen_workspace_size(_pp(T=100))
    assert _lib.prefill_varlen_workspace_size(_pp(T=100, dk=64, dv=64)) > 0
    assert _lib.prefill_varlen_workspace_size(_pp(T=100, flags=1)) == (_lib.prefill_varlen_workspace_size(_pp(T=100))
                                                                       + 2 * 100 * 2 * 128 * 2)  # T H packed rows
    assert _lib.prefill_resume_workspace_size(_pp(T=100, W=32), 0) > _lib.prefill_resume_workspace_size(_pp(T=100), 0)
    assert _lib.prefill_resume_workspace_size(_pp(T=100, dk=64, dv=64), 1) > 0
    assert _lib.prefill_resume_workspace_size(_pp(T=100, flags=1), 0) > _lib.prefill_resume_workspace_size(_pp(T=100), 0)


def test_handoff_contract():
    """Any seqlen is accepted (T = 100 is not a whole number of chunks);
    every pointer is required, written buffers are disjoint, and the
    workspace covers ceil(T / 64) chunks."""
    f = Fake()
    p = _pp(B=2, T=100, H=3)
    assert _lib.prefill_handoff_workspace_size(p) == 2 * 2 * 3 * (3 * 10 * 256 * 2 + 64 * 4)
    assert _handoff(p, f) == 6                                  # workspace missing
    assert _handoff(p, f, fill_out=None) == 1
    assert _handoff(p, f, buf_alpha=None) == 1
    o = f()
    assert _handoff(p, f, o=o, buf_k=o) == 5                    # buffer over an output
    k = f()
    assert _handoff(p, f, k=k, fill_out=k) == 5                 # output over an input
    assert _handoff(_pp(B=0, T=100), f) == 0                    # empty batch: no-op
    # the chunked call with T = 100 is the hand-over: same workspace
    assert _lib.prefill_workspace_size(p) == _lib.prefill_handoff_workspace_size(p)


def test_chunked_window_buffer_contract():
    """gdnq_prefill_chunked with decode's window buffer (or T not a multiple
    of the window) is the hand-over: all five buffer arguments required, GDN
    only, no state_f32, decode's window at most 64; its workspace size
    covers both forms when T is a multiple of the window."""
    f = Fake()
    bufs = lambda: dict(buf_k=f(), buf_v=f(), buf_alpha=f(), buf_beta=f(), fill_out=f())
    p = _pp(B=2, T=100, H=3)
    assert _prefill(p, f) == 1                                   # the open window needs the buffer
    assert _prefill(p, f, **bufs()) == 6                         # workspace missing (the hand-over's)
    b = bufs()
    b["fill_out"] = None
    assert _prefill(p, f, **b) == 1
    assert _prefill(p, f, state_f32=f(), **bufs()) == 2
    assert _prefill(_pp(B=2, T=128, H=3, dv=128, flags=2), f, beta=None, codes=None, scales=None,
                    state_f32=f(), **bufs()) == 8                # not for SSD
    assert _prefill(_pp(B=2, T=128, H=3, flags=8), f, codes=None, scales=None, **bufs()) == 8  # nor NO_REQUANT
    assert _prefill(_pp(B=2, T=256, H=3, W=128), f, **bufs()) == 2  # decode's window is at most 64
    # no windows without requantization or with SSD: any T, no buffer needed
    assert _prefill(_pp(B=2, T=100, H=3, flags=8), f, codes=None, scales=None) == 1  # (state_f32 missing)
    assert _prefill(_pp(B=2, T=100, H=3, flags=2, dv=64), f, beta=None, codes=None, scales=None) == 2  # (T % 64)
    p = _pp(B=2, T=128, H=3, W=32, C=32)
    assert _prefill(p, f, **bufs()) == 6                         # whole windows and the buffer: the hand-over
    need = _lib.prefill_workspace_size(p)
    assert need >= _lib.prefill_handoff_workspace_size(p) > 0
    assert _prefill(p, f, **bufs(), workspace=f(), ws=need - 1) == 6


def test_handoff_buffer_formats():
    """GDNQ_FLAG_BUF_BF16 / GDNQ_FLAG_BUF_FP8 select decode's window-buffer
    formats for the hand-over, varlen and resume calls and the chunked
    prefill given the window buffer (not without it).  The buffer spans follow the format: a buf_v placed right after
    a bf16-sized buf_k is disjoint from it under the bf16 flag and overlaps
    an fp32 buf_k; an FP8 buffer holds B H W d code bytes then B H W fp32
    scales."""
    B, T, H, d, W = 2, 100, 3, 128, 64
    for flags in (16, 32):
        p = _pp(B=B, T=T, H=H, flags=flags)
        ws = _lib.prefill_handoff_workspace_size(p)
        assert ws == _lib.prefill_handoff_workspace_size(_pp(B=B, T=T, H=H)) > 0
        assert _lib.prefill_varlen_workspace_size(p) > 0
        assert _lib.prefill_resume_workspace_size(p, 0) > 0
        pc = _pp(B=B, T=128, H=H, flags=flags)
        assert _lib.prefill_workspace_size(pc) == _lib.prefill_handoff_workspace_size(pc) > 0
        assert _prefill(pc, Fake()) == 8                         # a buffer format without the buffer
    f = Fake()
    k = f(1 << 26)
    o = f()
    wsp = f()
    ws = _lib.prefill_handoff_workspace_size(_pp(B=B, T=T, H=H))
    # bf16: buf_v right after a bf16 buf_k is fine (only the planted o / fill_out overlap is reported)
    st = _handoff(_pp(B=B, T=T, H=H, flags=16), f, buf_k=k, buf_v=k + B * H * W * d * 2, o=o, fill_out=o,
                  workspace=wsp, ws=ws)
    assert st == 5 and b"buf" not in L.gdnq_last_error(), L.gdnq_last_error()
    assert _handoff(_pp(B=B, T=T, H=H, flags=0), f, buf_k=k, buf_v=k + B * H * W * d * 2, workspace=wsp,
                    ws=ws) == 5
    assert b"buf_k overlaps buf_v" in L.gdnq_last_error() or b"buf_v overlaps buf_k" in L.gdnq_last_error()
    # FP8: codes then scales
    st = _handoff(_pp(B=B, T=T, H=H, flags=32), f, buf_k=k, buf_v=k + B * H * W * (d + 4), o=o, fill_out=o,
                  workspace=wsp, ws=ws)
    assert st == 5 and b"buf" not in L.gdnq_last_error(), L.gdnq_last_error()
    assert _handoff(_pp(B=B, T=T, H=H, flags=32), f, buf_k=k, buf_v=k + B * H * W * (d + 4) - 16, workspace=wsp,
                    ws=ws) == 5


# ---------------------------------------------------------------- variable-length prefill
def _varlen(params, fake, cu="fake", **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), beta=fake(), init_codes=None,
             init_scales=None, o=fake(), codes=fake(), scales=fake(), buf_k=fake(), buf_v=fake(),
             buf_alpha=fake(), buf_beta=fake(), fill_out=fake(), workspace=None, ws=0)
    a.update(over)
    cu = fake() if cu == "fake" else cu
    return _lib.prefill_varlen(params, cu, a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                               a["init_codes"], a["init_scales"], a["o"], a["codes"], a["scales"],
                               a["buf_k"], a["buf_v"], a["buf_alpha"], a["buf_beta"],
                               a["fill_out"], a["workspace"], a["ws"], None)


@pytest.mark.parametrize("params,status", [
    (_pp(W=65), 2), (_pp(W=0), 2), (_pp(C=8), 2), (_pp(dk=64, dv=128), 2), (_pp(ind=0), 3),
    (_pp(flags=8), 8), (_pp(dv=64, flags=2 | 1 | 4), 8),   # GDN only, requantizing
    (_pp(T=1 << 20, H=8192), 2),                           # the packed outputs past 4 GiB
])
def test_varlen_rejects_bad_params(params, status):
    assert _varlen(params, Fake()) == status
    assert _lib.prefill_varlen_workspace_size(params) == 0


def test_varlen_contract():
    """batch counts sequences and seqlen the packed tokens; the workspace
    bounds the chunks by floor(T / 64) + B per head and adds the sequence
    map; cu_seqlens is required and 4-byte aligned, and no written buffer
    may overlap it."""
    f = Fake()
    B, T, H = 5, 300, 3
    p = _pp(B=B, T=T, H=H)
    assert _lib.prefill_varlen_workspace_size(p) == (T // 64 + B) * H * (3 * 10 * 256 * 2 + 64 * 4) + (4 * B + 2) * 4
    ws = f()
    need = _lib.prefill_varlen_workspace_size(p)
    assert _varlen(p, f) == 6                                   # workspace missing
    assert _varlen(p, f, cu=None, workspace=ws, ws=need) == 1   # cu_seqlens missing
    assert _varlen(p, f, cu=f() + 2, workspace=ws, ws=need) == 4
    o = f()
    assert _varlen(p, f, cu=o, o=o, workspace=ws, ws=need) == 5
    assert _varlen(p, f, fill_out=None, workspace=ws, ws=need) == 1
    assert _varlen(_pp(B=0, T=0), f, cu=None) == 0              # no sequences: no-op


def test_output_offset_bound_counts_padding():
    """Outputs are addressed with 32-bit byte offsets, and the last partial
    chunk's padding tokens are addressed too (their stores are dropped): the
    limit is (T + 64) H 512 bytes < 4 GiB."""
    assert _lib.prefill_handoff_workspace_size(_pp(T=(1 << 23) - 64, H=1)) == 0
    assert _lib.prefill_handoff_workspace_size(_pp(T=(1 << 23) - 128, H=1)) > 0


# ---------------------------------------------------------------- resuming from decode
def _resume(params, fake, cu=None, fill_in="fake", **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), beta=fake(), o=fake(), codes=fake(),
             scales=fake(), buf_k=fake(), buf_v=fake(), buf_alpha=fake(), buf_beta=fake(),
             fill_out=fake(), workspace=None, ws=0)
    a.update(over)
    fi = fake() if fill_in == "fake" else fill_in
    return _lib.prefill_resume(params, cu, fi, a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["o"],
                               a["codes"], a["scales"], a["buf_k"], a["buf_v"], a["buf_alpha"],
                               a["buf_beta"], a["fill_out"], a["workspace"], a["ws"], None)


@pytest.mark.parametrize("params,status", [
    (_pp(W=65), 2), (_pp(W=0), 2), (_pp(C=8), 2), (_pp(dk=64, dv=128), 2), (_pp(ind=0), 3),
    (_pp(flags=8), 8), (_pp(dv=64, flags=2 | 1 | 4), 8),   # GDN only, requantizing
    (_pp(B=1 << 16, T=1 << 16), 2),                        # 2^32 new tokens
])
def test_resume_rejects_bad_params(params, status):
    assert _resume(params, Fake()) == status
    assert _lib.prefill_resume_workspace_size(params, 0) == 0


def test_resume_contract():
    """The workspace bounds the chunks by floor(N / 64) + 2 B per head for N
    new tokens (a prefix adds at most one chunk per sequence), plus chunk 0
    of every sequence staged and the sequence map; fill_in is required and
    may be fill_out itself but no other written buffer; the stored state is
    required."""
    f = Fake()
    B, T, H = 3, 100, 2
    p = _pp(B=B, T=T, H=H)
    stage = B * 64 * H * (3 * 128 * 2 + 2 * 4)
    need = (B * T // 64 + 2 * B) * H * (3 * 10 * 256 * 2 + 64 * 4) + stage + (4 * B + 2) * 4
    assert _lib.prefill_resume_workspace_size(p, 0) == need
    need_v = (T // 64 + 2 * B) * H * (3 * 10 * 256 * 2 + 64 * 4) + stage + (4 * B + 2) * 4
    assert _lib.prefill_resume_workspace_size(p, 1) == need_v
    ws = f()
    assert _resume(p, f) == 6                                    # workspace missing
    assert _resume(p, f, fill_in=None, workspace=ws, ws=need) == 1
    assert _resume(p, f, fill_in=f() + 2, workspace=ws, ws=need) == 4
    o = f()
    assert _resume(p, f, fill_in=o, o=o, workspace=ws, ws=need) == 5
    fo = f()
    assert _resume(p, f, fill_in=fo, fill_out=fo) == 6           # same array: past the alias checks
    assert _resume(p, f, codes=None, workspace=ws, ws=need) == 1
    assert _resume(_pp(B=0, T=0), f) == 0                       # no sequences: no-op


def test_prefill_noalloc_refuses_more_than_its_array():
    """gdnq_prefill_chunked_noalloc: a call whose workspace would exceed the
    library's device scratch array is refused during validation (fake
    pointers: nothing is looked up or launched); the reason names the limit."""
    fake = Fake()
    p = _lib.PrefillParams(4, 8192, 16, 128, 128, 64, 64, 1, 1, 0)
    assert L.gdnq_prefill_workspace_size(p) > _lib.NOALLOC_SCRATCH_BYTES
    big = [fake(1 << 30) for _ in range(6)]  # q, k, v, alpha, beta, o: disjoint spans
    st = _lib.prefill_chunked_noalloc(p, *big[:5], None, None, big[5], fake(), fake(), None, None)
    assert st == 6
    assert b"allocation-free" in L.gdnq_last_error()
    # the same shapes with a workspace argument are accepted up to the pointer checks
    p_ok = _lib.PrefillParams(1, 128, 2, 128, 128, 64, 64, 1, 1, 0)
    assert L.gdnq_prefill_workspace_size(p_ok) <= _lib.NOALLOC_SCRATCH_BYTES
    assert _lib.prefill_chunked_noalloc(p_ok, None, fake(), fake(), fake(), fake(), None, None, fake(),
                                        fake(), fake(), None, None) == 1  # q is NULL
