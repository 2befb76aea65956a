"""Runs oracle calls in worker processes for the full-size GPU tests.

The workers are started with "spawn" and import only numpy and the oracle:
they never touch the GPU.  Each task is one self-contained oracle call whose
inputs (including the GPU's state before the window) travel with it."""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

WORKERS = min(8, os.cpu_count() or 1)


def _prefill_window(args):
    import oracle as O
    xs, codes0, scale0, W, qmax = args
    r = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], W=W, codes0=codes0,
                  scale0=scale0, qmax=qmax)
    return r["o"], r["codes"], r["scale"]


def _ssd_sequence(args):
    import oracle as O
    xs, = args
    r = O.prefill(xs["q"], xs["k"], xs["v"], xs["alpha"], None, W=None, kind="ssd", rot=True,
                  qk_int8=True)
    return r["o"], r["S"]


def _decode_close(args):
    import oracle as O
    x, before, W = args
    _, rc, rs, *_ = O.decode_step(*x, *before, W)
    return rc, rs


_FUNCS = {"prefill_window": _prefill_window, "ssd_sequence": _ssd_sequence,
          "decode_close": _decode_close}


def pool():
    return cf.ProcessPoolExecutor(max_workers=WORKERS, mp_context=mp.get_context("spawn"))


def submit(ex, kind, *args):
    return ex.submit(_FUNCS[kind], args)
