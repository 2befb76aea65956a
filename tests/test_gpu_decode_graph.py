"""Decode steps captured into a HIP graph (how the benchmark times them, and
how a serving loop replays a captured step) against the same steps launched
eagerly, through the C ABI.

Two identical decode states; 8 steps of one are captured once (bound
launchers on a side stream, each step writing its own output buffer) and
the graph is replayed three times, with the other state stepping eagerly
and the host synchronizing between replays.  After every replay all eight
outputs and the whole state (codes, scales, window buffer, fills) equal the
eager ones bitwise.  The decode launch records no memset, so the graph holds
kernel nodes only.
"""

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


@pytest.mark.parametrize("W,buf", [(16, torch.float32), (8, torch.bfloat16)])
def test_decode_graph_replays_match_eager(W, buf):
    B, H, d, K, R = 8, 4, 128, 8, 3
    x = wl.decode_batch(B=B, H=H, dk=d, dv=d, W=W, seed=17, poison=False)
    codes, scales = O.quantize_rows(x["state"])

    def make():
        st = ops.DecodeState(dev(codes), dev(scales), W, fill=dev(x["fill"]), buf_dtype=buf)
        st.buf_k.copy_(dev(x["buf_k"]).to(buf))
        st.buf_v.copy_(dev(x["buf_v"]).to(buf))
        st.buf_alpha.copy_(dev(x["buf_alpha"]))
        st.buf_beta.copy_(dev(x["buf_beta"]))
        return st

    eager, graphed = make(), make()
    toks = []
    for t in range(4):
        y = wl.decode_tokens(B=B, H=H, dk=d, dv=d, step=t, seed=18)
        toks.append([dev(y["q"], torch.bfloat16), dev(y["k"], torch.bfloat16), dev(y["v"], torch.bfloat16),
                     dev(y["alpha"]), dev(y["beta"])])
    outs = [torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV) for _ in range(K)]
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        launch = [graphed.bind(*toks[i % 4], o=outs[i]) for i in range(K)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for i in range(K):
            launch[i]()
    torch.cuda.synchronize()
    for r in range(R):
        print(f"W={W} {buf}: replay {r}", flush=True)
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        ref = [eager.step(*toks[i % 4]) for i in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            assert torch.equal(outs[i], ref[i]), (r, i)
        for name in STATE:
            a, b = getattr(graphed, name), getattr(eager, name)
            if name == "fill":  # K is even: the fill ping-pong is back where it started
                assert torch.equal(a, b), (r, name)
            else:
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (r, name)
    assert int(host(eager.fill).max()) < W
