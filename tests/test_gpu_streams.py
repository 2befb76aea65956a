"""Calls on several streams at once.  The decode step keeps no state of its
own between calls (its head pool is in LDS) and the prefill's workspace is
the caller's, so two decode states stepped on two streams while a GDN and an
SSD prefill run on a third give bitwise the results of the same calls made
one after another on one stream."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_util import DEV, dev, host

pytestmark = pytest.mark.gpu

if DEV is not None:
    from quantized_recurrent_state_gdnq_amd import ops

STATE = ("codes", "scales", "buf_k", "buf_v", "buf_alpha", "buf_beta", "fill")


def _decode_setup(seed, B=16, H=8, d=128, W=16):
    x = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=seed, poison=False)
    codes, scales = O.quantize_rows(x["state"])

    def make():
        st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(x["fill"]))
        st.buf_k.copy_(dev(x["buf_k"]))
        st.buf_v.copy_(dev(x["buf_v"]))
        st.buf_alpha.copy_(dev(x["buf_alpha"]))
        st.buf_beta.copy_(dev(x["buf_beta"]))
        return st

    toks = []
    for t in range(6):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=seed + 1)
        toks.append([dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16), dev(y["v"], torch.bfloat16),
                     dev(y["alpha"]), dev(y["beta"])])
    return make, toks


def _prefill_inputs(seed):
    g = wl.gdn_prefill(B=2, T=256, H=4, dk=128, dv=128, seed=seed)
    s = wl.ssd_prefill(B=1, T=256, H=6, dk=128, dv=64, seed=seed + 1)
    gi = [dev(g["q"], torch.bfloat16), dev(g["k"], torch.bfloat16), dev(g["v"], torch.bfloat16),
          dev(g["alpha"]), dev(g["beta"])]
    si = [dev(s["q"], torch.bfloat16), dev(s["k"], torch.bfloat16), dev(s["v"], torch.bfloat16), dev(s["alpha"])]
    return gi, si


def _run(make_a, toks_a, make_b, toks_b, gi, si, streams):
    """Six steps of each decode state and the two prefills; streams = None
    runs everything on the current stream in that order."""
    a, b = make_a(), make_b()
    torch.cuda.synchronize()
    sa, sb, sp = streams if streams else (None, None, None)
    oa, ob, pre = [], [], {}

    def on(s):
        return torch.cuda.stream(s) if s is not None else torch.cuda.stream(torch.cuda.current_stream())

    for i in range(6):
        with on(sa):
            oa.append(a.step(*toks_a[i]))
        with on(sb):
            ob.append(b.step(*toks_b[i]))
        if i == 2:
            with on(sp):
                pre["gdn"] = ops.prefill_chunked(*gi, out_dtype=torch.float32)
                pre["ssd"] = ops.prefill_chunked(*si, None, ssd=True, int8_qk=True, wht=True,
                                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    res = {"oa": [host(t) for t in oa], "ob": [host(t) for t in ob]}
    for name, st in (("a", a), ("b", b)):
        for f in STATE:
            res[f"{name}.{f}"] = host(getattr(st, f))
    res["gdn"] = [host(t) for t in pre["gdn"]]
    res["ssd"] = [host(t) for t in pre["ssd"]]
    return res


def test_concurrent_streams_match_one_stream():
    make_a, toks_a = _decode_setup(31)
    make_b, toks_b = _decode_setup(41)
    gi, si = _prefill_inputs(51)
    ref = _run(make_a, toks_a, make_b, toks_b, gi, si, None)
    streams = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    for rep in range(2):
        got = _run(make_a, toks_a, make_b, toks_b, gi, si, streams)
        for key, want in ref.items():
            have = got[key]
            if isinstance(want, list):
                for i, (w, h) in enumerate(zip(want, have)):
                    assert np.array_equal(w, h, equal_nan=True), f"run {rep}: {key}[{i}] differs"
            else:
                assert np.array_equal(want, have, equal_nan=True), f"run {rep}: {key} differs"
