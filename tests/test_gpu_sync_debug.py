"""GDNQ_SYNC_DEBUG=1: every call synchronizes its stream before it returns.

A child process loads the library with the variable set and makes a codec
call, a decode step and a GDN prefill; its results must equal, bitwise, the
same calls made asynchronously in this process (the mode changes when a call
returns, not what it computes).
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from quantized_recurrent_state_gdnq_amd import _lib, ops

from gpu_util import DEV, dev

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _calls():
    """The three calls on seeded inputs; returns host arrays."""
    x = wl.decode_batch(B=4, H=3, W=8, seed=11, poison=False)
    codes, scales = ops.quantize_state(dev(x["state"]))
    ci, si = codes.clone(), scales.clone()
    fo = torch.empty(4, dtype=torch.int32, device=DEV)
    bk, bv, ba, bb = (dev(x[n]) for n in ("buf_k", "buf_v", "buf_alpha", "buf_beta"))
    o = ops.decode_step(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16), dev(x["v"], torch.bfloat16),
                        dev(x["alpha"]), dev(x["beta"]), codes, scales, bk, bv, ba, bb,
                        dev(x["fill"]), fo, out_dtype=torch.float32)
    p = wl.gdn_prefill(B=1, T=256, H=2, seed=12)
    po, pc, ps = ops.prefill_chunked(*(dev(p[n], torch.bfloat16) for n in ("q", "k", "v")),
                                     dev(p["alpha"]), dev(p["beta"]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    out = {"qcodes": ci, "qscales": si, "o": o, "codes": codes, "scales": scales, "fill": fo,
           "buf_k": bk, "po": po, "pc": pc, "ps": ps}
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_sync_debug_calls_match_async(tmp_path):
    assert _lib.lib.gdnq_sync_debug() == 0
    ref = _calls()
    out = tmp_path / "sync.npz"
    code = ("import sys; sys.path.insert(0, 'tests'); import numpy as np; "
            "from quantized_recurrent_state_gdnq_amd import _lib; assert _lib.lib.gdnq_sync_debug() == 1; "
            "import test_gpu_sync_debug as t; np.savez(sys.argv[1], **t._calls()); print('child ok', flush=True)")
    env = dict(os.environ, GDNQ_SYNC_DEBUG="1")
    print("child: GDNQ_SYNC_DEBUG=1, codec + decode B=4 H=3 W=8 + prefill B=1 T=256 H=2", flush=True)
    r = subprocess.run([sys.executable, "-c", code, str(out)], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=240)
    assert r.returncode == 0 and "child ok" in r.stdout, r.stderr[-3000:]
    got = np.load(out)
    for k, v in ref.items():
        assert np.array_equal(got[k], v, equal_nan=True), k
