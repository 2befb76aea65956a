"""Helpers for the GPU parity tests: device transfer, guard canaries and the
parity metrics (the same bar for every kernel).

Parity bar:
  * outputs: max relative error per output vector, max_r |d_r| / max_r |ref_r|,
    maximised over vectors: <= 1e-3 with fp32 inputs, <= 2e-2 with bf16 inputs;
  * int8 codes that were requantized: |diff| <= 1 everywhere and nonzero on at
    most 0.1% of them; codes that must not change: bitwise;
  * scales: |d| / ref <= 1e-5 where ref > 0, exact where ref == 0;
  * integer bookkeeping (fills) and copied data (buffer appends): bitwise.

The code and scale bars bound one requantization (both sides requantize the
same state): tests gate them teacher-forced.  Free-running comparisons over
many windows are diagnostics; their scales are held to FREE_SCALE_DRIFT (two
code units of the row absmax), and the drift measured is printed.
"""

import numpy as np
import torch

OUT_TOL_F32 = 1e-3
OUT_TOL_BF16 = 2e-2
CODE_FLIP_FRAC = 1e-3
SCALE_RTOL = 1e-5
FREE_SCALE_DRIFT = 2.0 / 127.0

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return t if dtype is None else t.to(dtype)


def host(t):
    if t.dtype in (torch.bfloat16, torch.float8_e4m3fn):
        t = t.float()
    return t.detach().cpu().numpy()


class Guarded:
    """A contiguous tensor view with canary-filled guard zones on both sides
    (detects out-of-bounds writes by a kernel)."""

    PAD = 4096  # elements, keeps the view 16-byte aligned for every dtype used

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape))
        self.n = n
        self.dtype = dtype
        self.flat = torch.empty(n + 2 * self.PAD, dtype=dtype, device=DEV)
        canary = -77 if dtype in (torch.int8, torch.int32) else float("nan") if fill is None else fill
        self.canary = canary
        self.flat.fill_(canary)
        self.t = self.flat[self.PAD:self.PAD + n].view(shape)

    def set(self, x):
        self.t.copy_(x if isinstance(x, torch.Tensor) else dev(x).to(self.dtype))
        return self

    def guards_intact(self):
        g = torch.cat([self.flat[:self.PAD], self.flat[self.PAD + self.n:]])
        if self.dtype.is_floating_point and np.isnan(self.canary):
            return bool(torch.isnan(g).all())
        return bool((g == self.canary).all())


def max_rel_err(out, ref):
    """Max over output vectors (last axis) of max|out - ref| / max|ref|."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(np.max(rel)) if rel.size else 0.0


def code_stats(got, ref):
    d = np.abs(np.asarray(got, np.int32) - np.asarray(ref, np.int32))
    return (float(np.mean(d != 0)) if d.size else 0.0), (int(d.max()) if d.size else 0)


def assert_codes(got, ref, what=""):
    frac, mx = code_stats(got, ref)
    assert mx <= 1, f"{what}: a code differs by {mx}"
    assert frac <= CODE_FLIP_FRAC, f"{what}: {frac:.4%} of codes differ (limit 0.1%)"
    return frac


def assert_scales(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    zero = ref == 0
    assert np.array_equal(got[zero], ref[zero]), f"{what}: zero-row scales differ"
    if np.any(~zero):
        rel = np.max(np.abs(got[~zero] - ref[~zero]) / ref[~zero])
        assert rel <= SCALE_RTOL, f"{what}: scale relative error {rel:.3e}"


def assert_free_scales(got, ref, what=""):
    """Free-running scale drift: max |d| / ref over rows with ref > 0, zero
    rows exactly; printed, and held to FREE_SCALE_DRIFT."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    zero = ref == 0
    assert np.array_equal(got[zero], ref[zero]), f"{what}: zero-row scales differ"
    rel = float(np.max(np.abs(got[~zero] - ref[~zero]) / ref[~zero])) if np.any(~zero) else 0.0
    frac = float(np.mean(np.abs(got[~zero] - ref[~zero]) > SCALE_RTOL * ref[~zero])) if np.any(~zero) else 0.0
    print(f"free-running scale drift {what}: max {rel:.3e}, rows beyond 1e-5 {frac:.3%}")
    assert rel <= FREE_SCALE_DRIFT, f"{what}: free-running scale drift {rel:.3e}"
    return rel
