"""The allocation-free prefill entry point, gdnq_prefill_chunked_noalloc,
called through the C ABI: its workspace is the library's device scratch
array instead of a caller's buffer.  Its results must equal those of
gdnq_prefill_chunked with a workspace (the same kernels), bitwise, on two
calls in a row whose second is smaller than the first (the array keeps the
first call's contents), for the GDN recurrence (8- and 4-bit state) and for
the SSD recurrence with rotated int8 operands.  A call too large for the
array is refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import _lib, ops


def _t(x, dt=None):
    y = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return y if dt is None else y.to(dt)


def _gdn(B, T, H, seed, state_bits):
    x = wl.gdn_prefill(B=B, T=T, H=H, dk=128, dv=128, seed=seed)
    g = np.random.default_rng(seed + 1)
    c0 = torch.from_numpy(g.integers(-7 if state_bits == 4 else -127, 8 if state_bits == 4 else 128,
                                     (B, H, 128, 128 * state_bits // 8)).astype(np.int8)).to(DEV)
    s0 = _t((g.uniform(0.001, 0.01, (B, H, 128))).astype(np.float32))
    ins = [_t(x["q"], torch.bfloat16), _t(x["k"], torch.bfloat16), _t(x["v"], torch.bfloat16),
           _t(x["alpha"]), _t(x["beta"])]
    outs = []
    for noalloc in (False, True):
        o = torch.empty((B, T, H, 128), dtype=torch.float32, device=DEV)
        codes = torch.empty((B, H, 128, 128 * state_bits // 8), dtype=torch.int8, device=DEV)
        scales = torch.empty((B, H, 128), dtype=torch.float32, device=DEV)
        p = ops._prefill_params(ins[0], ins[2], window=64, chunk=64, wht=False, ssd=False, int8_qk=False,
                                out_dtype=torch.float32, state_bits=state_bits)
        ptr = [t.data_ptr() for t in ins]
        if noalloc:
            st = _lib.prefill_chunked_noalloc(p, *ptr, c0.data_ptr(), s0.data_ptr(), o.data_ptr(),
                                              codes.data_ptr(), scales.data_ptr(), None,
                                              torch.cuda.current_stream().cuda_stream)
        else:
            ws = torch.empty(_lib.prefill_workspace_size(p), dtype=torch.uint8, device=DEV)
            st = _lib.prefill_chunked(p, *ptr, c0.data_ptr(), s0.data_ptr(), o.data_ptr(), codes.data_ptr(),
                                      scales.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                      torch.cuda.current_stream().cuda_stream)
        _lib.check(st)
        outs.append((o, codes, scales))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("state_bits", [8, 4])
def test_noalloc_gdn_two_calls_second_smaller(state_bits):
    for B, T, H, seed in ((2, 512, 5, 1), (1, 128, 2, 2)):  # 40 chunk-heads, then 4
        (o0, c0, s0), (o1, c1, s1) = _gdn(B, T, H, seed, state_bits)
        assert torch.equal(o0, o1), (B, T, H)
        assert torch.equal(c0, c1) and torch.equal(s0, s1), (B, T, H)


def test_noalloc_gdn_at_its_limit():
    """B=1, T=8192, H=33: 4224 chunk-heads, 66.0 MB of workspace, just
    within the array (4297 chunk-heads)."""
    (o0, c0, s0), (o1, c1, s1) = _gdn(1, 8192, 33, 5, 8)
    assert torch.equal(o0, o1) and torch.equal(c0, c1) and torch.equal(s0, s1)


def _ssd(B, T, H, seed):
    x = wl.ssd_prefill(B=B, T=T, H=H, dk=128, dv=64, seed=seed)
    q, k, v = (_t(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    a = _t(x["alpha"])
    r0 = ops.prefill_chunked(q, k, v, a, None, ssd=True, wht=True, int8_qk=True, out_dtype=torch.float32)
    o = torch.empty((B, T, H, 64), dtype=torch.float32, device=DEV)
    S = torch.empty((B, H, 64, 128), dtype=torch.float32, device=DEV)
    r1 = ops.prefill_chunked(q, k, v, a, None, ssd=True, wht=True, int8_qk=True, out_dtype=torch.float32,
                             o=o, state_f32=S, noalloc=True)
    torch.cuda.synchronize()
    return r0, r1


def test_noalloc_ssd_two_calls_second_smaller():
    for B, T, H, seed in ((2, 1024, 40, 3), (1, 128, 3, 4)):
        (o0, S0), (o1, S1) = _ssd(B, T, H, seed)
        assert torch.equal(o0, o1) and torch.equal(S0, S1), (B, T, H)


def test_noalloc_refuses_more_than_its_array():
    """B=4, T=8192, H=16 needs 128 MB of workspace: refused, nothing written."""
    B, T, H = 4, 8192, 16
    q = torch.zeros((B, T, H, 128), dtype=torch.bfloat16, device=DEV)
    a = torch.ones((B, T, H), dtype=torch.float32, device=DEV)
    o = torch.full((B, T, H, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    codes = torch.full((B, H, 128, 128), 5, dtype=torch.int8, device=DEV)
    scales = torch.full((B, H, 128), 5.0, dtype=torch.float32, device=DEV)
    p = ops._prefill_params(q, q, window=64, chunk=64, wht=False, ssd=False, int8_qk=False,
                            out_dtype=torch.bfloat16)
    assert _lib.prefill_workspace_size(p) > _lib.NOALLOC_SCRATCH_BYTES
    st = _lib.prefill_chunked_noalloc(p, q.data_ptr(), q.data_ptr(), q.data_ptr(), a.data_ptr(), a.data_ptr(),
                                      None, None, o.data_ptr(), codes.data_ptr(), scales.data_ptr(), None,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 6  # GDNQ_ERR_WORKSPACE
    assert b"allocation-free" in _lib.lib.gdnq_last_error()
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((codes == 5).all()) and bool((scales == 5.0).all())
