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
    (_p(ind=2), 3), (_p(outd=5), 3), (_p(flags=2), 8), (_p(flags=4), 8), (_p(flags=128), 8),
    (_p(flags=16 | 2), 8), (_p(flags=16 | 32), 8),
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
             workspace=None, ws=0)
    a.update(over)
    return _lib.prefill_chunked(params, a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                a["init_codes"], a["init_scales"], a["o"], a["codes"],
                                a["scales"], a["state_f32"], a["workspace"], a["ws"], None)


@pytest.mark.parametrize("params,status", [
    (_pp(C=32, W=32), 2), (_pp(T=100), 2), (_pp(dk=64, dv=64), 2), (_pp(W=128), 2),
    (_pp(ind=0), 3), (_pp(outd=3), 3), (_pp(flags=4), 8), (_pp(flags=8), 8), (_pp(flags=16), 8),
    (_pp(flags=32), 8),
    (_pp(flags=1), 8),                   # GDN prefill takes no rotation flag
    (_pp(dv=64, flags=2 | 1), 8),        # SSD rotation only on the way to int8 operands
])
def test_prefill_rejects_bad_params(params, status):
    assert _prefill(params, Fake()) == status


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
    assert _prefill(_pp(dk=64, dv=64, flags=2), f, beta=None, codes=None, scales=None,
                    state_f32=f()) == 2


def test_workspace_size_is_queryable():
    assert L.gdnq_prefill_workspace_size(None) == 0
    p = _pp()
    assert _lib.prefill_workspace_size(p) >= 0


def test_workspace_sizes():
    """GDN: per chunk-head, T as three bf16 planes (24 KiB) and g (256 B);
    SSD int8: codes and scales of q and k per token row; plain SSD: none."""
    B, T, H = 2, 256, 3
    nch = B * (T // 64) * H
    assert _lib.prefill_workspace_size(_pp(B=B, T=T, H=H)) == nch * (3 * 64 * 64 * 2 + 64 * 4)
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
    (_pp(C=32, W=32), 2), (_pp(dk=64, dv=64), 2), (_pp(W=128), 2), (_pp(ind=0), 3),
    (_pp(flags=1), 8), (_pp(dv=64, flags=2 | 1 | 4), 8),   # GDN only
    (_pp(T=1 << 20, H=8192), 2),                           # one sequence's outputs past 4 GiB
])
def test_handoff_rejects_bad_params(params, status):
    assert _handoff(params, Fake()) == status


def test_handoff_contract():
    """Any seqlen is accepted (T = 100 is not a whole number of chunks);
    every pointer is required, written buffers are disjoint, and the
    workspace covers ceil(T / 64) chunks."""
    f = Fake()
    p = _pp(B=2, T=100, H=3)
    assert _lib.prefill_handoff_workspace_size(p) == 2 * 2 * 3 * (3 * 64 * 64 * 2 + 64 * 4)
    assert _handoff(p, f) == 6                                  # workspace missing
    assert _handoff(p, f, fill_out=None) == 1
    assert _handoff(p, f, buf_alpha=None) == 1
    o = f()
    assert _handoff(p, f, o=o, buf_k=o) == 5                    # buffer over an output
    k = f()
    assert _handoff(p, f, k=k, fill_out=k) == 5                 # output over an input
    assert _handoff(_pp(B=0, T=100), f) == 0                    # empty batch: no-op
    assert _lib.prefill_workspace_size(p) == 0                  # the chunked prefill rejects T = 100


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
    (_pp(C=32, W=32), 2), (_pp(dk=64, dv=64), 2), (_pp(ind=0), 3),
    (_pp(flags=1), 8), (_pp(dv=64, flags=2 | 1 | 4), 8),   # GDN only
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
    assert _lib.prefill_varlen_workspace_size(p) == (T // 64 + B) * H * (3 * 64 * 64 * 2 + 64 * 4) + (4 * B + 2) * 4
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
    (_pp(C=32, W=32), 2), (_pp(dk=64, dv=64), 2), (_pp(ind=0), 3),
    (_pp(flags=1), 8), (_pp(dv=64, flags=2 | 1 | 4), 8),   # GDN only
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
    need = (B * T // 64 + 2 * B) * H * (3 * 64 * 64 * 2 + 64 * 4) + stage + (4 * B + 2) * 4
    assert _lib.prefill_resume_workspace_size(p, 0) == need
    need_v = (T // 64 + 2 * B) * H * (3 * 64 * 64 * 2 + 64 * 4) + stage + (4 * B + 2) * 4
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
