"""ctypes binding of libgdnq.so (the C ABI declared in include/gdnq.h).

Argument marshalling only.  The shared library is loaded from this package's
directory (or from the path in GDNQ_LIBRARY, which the host-sanitizer test
uses for its instrumented build); if it is missing, importing this module
raises -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GDNQ_LIBRARY") or os.path.join(_HERE, "libgdnq.so")

GDNQ_OK = 0
STATUS_NAMES = {0: "GDNQ_OK", 1: "GDNQ_ERR_NULL", 2: "GDNQ_ERR_SHAPE", 3: "GDNQ_ERR_DTYPE",
                4: "GDNQ_ERR_ALIGN", 5: "GDNQ_ERR_ALIAS", 6: "GDNQ_ERR_WORKSPACE",
                7: "GDNQ_ERR_HIP", 8: "GDNQ_ERR_FLAGS"}
GDNQ_F32, GDNQ_BF16 = 0, 1
GDNQ_FLAG_WHT, GDNQ_FLAG_SSD, GDNQ_FLAG_INT8_QK, GDNQ_FLAG_BUF_BF16, GDNQ_FLAG_BUF_FP8 = 1, 2, 4, 16, 32
GDNQ_FLAG_STATE_4BIT = 64
GDNQ_FLAG_NO_REQUANT = 8
GDNQ_MAX_WINDOW = 1 << 24
GDNQ_FLAG_SLIDING = 128

# Every function the header declares.
EXPORTS = ("gdnq_quantize_state", "gdnq_decode_step", "gdnq_prefill_workspace_size",
           "gdnq_prefill_chunked", "gdnq_prefill_chunked_noalloc", "gdnq_prefill_handoff_workspace_size", "gdnq_prefill_handoff",
           "gdnq_prefill_varlen_workspace_size", "gdnq_prefill_varlen",
           "gdnq_prefill_resume_workspace_size", "gdnq_prefill_resume",
           "gdnq_decode_set_schedule", "gdnq_status_string", "gdnq_last_error", "gdnq_version",
           "gdnq_sync_debug")


class DecodeParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("window", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class PrefillParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("window", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class GdnqError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


def _load():
    # A process must hold a single HIP runtime.  PyTorch ships its own copy
    # (same soname); importing torch first makes libgdnq bind to that copy
    # instead of pulling in a second runtime from /opt/rocm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -m quantized_recurrent_state_gdnq_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_size_t
    lib.gdnq_quantize_state.argtypes = [vp, i64, i32, vp, vp, u32, vp]
    lib.gdnq_quantize_state.restype = i32
    lib.gdnq_decode_step.argtypes = [ctypes.POINTER(DecodeParams)] + [vp] * 15
    lib.gdnq_decode_step.restype = i32
    lib.gdnq_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    lib.gdnq_prefill_workspace_size.restype = sz
    lib.gdnq_prefill_chunked.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 17 + [sz, vp]
    lib.gdnq_prefill_chunked.restype = i32
    lib.gdnq_prefill_chunked_noalloc.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 17
    lib.gdnq_prefill_chunked_noalloc.restype = i32
    lib.gdnq_prefill_handoff_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    lib.gdnq_prefill_handoff_workspace_size.restype = sz
    lib.gdnq_prefill_handoff.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 16 + [sz, vp]
    lib.gdnq_prefill_handoff.restype = i32
    lib.gdnq_prefill_varlen_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
    lib.gdnq_prefill_varlen_workspace_size.restype = sz
    lib.gdnq_prefill_varlen.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 17 + [sz, vp]
    lib.gdnq_prefill_varlen.restype = i32
    lib.gdnq_prefill_resume_workspace_size.argtypes = [ctypes.POINTER(PrefillParams), i32]
    lib.gdnq_prefill_resume_workspace_size.restype = sz
    lib.gdnq_prefill_resume.argtypes = [ctypes.POINTER(PrefillParams)] + [vp] * 16 + [sz, vp]
    lib.gdnq_prefill_resume.restype = i32
    lib.gdnq_decode_set_schedule.argtypes = [i32, i32]
    lib.gdnq_decode_set_schedule.restype = i32
    lib.gdnq_status_string.argtypes = [i32]
    lib.gdnq_status_string.restype = ctypes.c_char_p
    lib.gdnq_last_error.argtypes = []
    lib.gdnq_last_error.restype = ctypes.c_char_p
    lib.gdnq_version.argtypes = []
    lib.gdnq_version.restype = i32
    lib.gdnq_sync_debug.argtypes = []
    lib.gdnq_sync_debug.restype = i32
    return lib


lib = _load()


def check(status):
    if status != GDNQ_OK:
        raise GdnqError(status, lib.gdnq_last_error().decode())
    return status


def decode_set_schedule(grid, open_waves):
    return lib.gdnq_decode_set_schedule(grid, open_waves)


def quantize_state(S, rows, d_k, codes, scales, flags, stream):
    return lib.gdnq_quantize_state(S, rows, d_k, codes, scales, flags, stream)


def decode_step(params, q, k, v, alpha, beta, codes, scales, buf_k, buf_v, buf_alpha, buf_beta,
                fill_in, fill_out, o, stream):
    return lib.gdnq_decode_step(ctypes.byref(params), q, k, v, alpha, beta, codes, scales, buf_k,
                                buf_v, buf_alpha, buf_beta, fill_in, fill_out, o, stream)


def prefill_workspace_size(params):
    return lib.gdnq_prefill_workspace_size(ctypes.byref(params))


def prefill_chunked(params, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales,
                    state_f32, workspace, workspace_bytes, stream, buf_k=None, buf_v=None, buf_alpha=None,
                    buf_beta=None, fill_out=None):
    """gdnq_prefill_chunked; the window-buffer pointers come last here (they
    sit before the workspace in the C signature)."""
    return lib.gdnq_prefill_chunked(ctypes.byref(params), q, k, v, alpha, beta, init_codes,
                                    init_scales, o, codes, scales, state_f32, buf_k, buf_v, buf_alpha,
                                    buf_beta, fill_out, workspace, workspace_bytes, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20  # GDNQ_NOALLOC_SCRATCH_BYTES


def prefill_chunked_noalloc(params, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales,
                            state_f32, stream, buf_k=None, buf_v=None, buf_alpha=None, buf_beta=None,
                            fill_out=None):
    return lib.gdnq_prefill_chunked_noalloc(ctypes.byref(params), q, k, v, alpha, beta, init_codes,
                                            init_scales, o, codes, scales, state_f32, buf_k, buf_v,
                                            buf_alpha, buf_beta, fill_out, stream)


def prefill_handoff_workspace_size(params):
    return lib.gdnq_prefill_handoff_workspace_size(ctypes.byref(params))


def prefill_handoff(params, q, k, v, alpha, beta, init_codes, init_scales, o, codes, scales,
                    buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream):
    return lib.gdnq_prefill_handoff(ctypes.byref(params), q, k, v, alpha, beta, init_codes,
                                    init_scales, o, codes, scales, buf_k, buf_v, buf_alpha,
                                    buf_beta, fill_out, workspace, workspace_bytes, stream)


def prefill_varlen_workspace_size(params):
    return lib.gdnq_prefill_varlen_workspace_size(ctypes.byref(params))


def prefill_varlen(params, cu_seqlens, q, k, v, alpha, beta, init_codes, init_scales, o, codes,
                   scales, buf_k, buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes,
                   stream):
    return lib.gdnq_prefill_varlen(ctypes.byref(params), cu_seqlens, q, k, v, alpha, beta,
                                   init_codes, init_scales, o, codes, scales, buf_k, buf_v,
                                   buf_alpha, buf_beta, fill_out, workspace, workspace_bytes,
                                   stream)


def prefill_resume_workspace_size(params, varlen):
    return lib.gdnq_prefill_resume_workspace_size(ctypes.byref(params), int(varlen))


def prefill_resume(params, cu_seqlens, fill_in, q, k, v, alpha, beta, o, codes, scales, buf_k,
                   buf_v, buf_alpha, buf_beta, fill_out, workspace, workspace_bytes, stream):
    return lib.gdnq_prefill_resume(ctypes.byref(params), cu_seqlens, fill_in, q, k, v, alpha, beta,
                                   o, codes, scales, buf_k, buf_v, buf_alpha, buf_beta, fill_out,
                                   workspace, workspace_bytes, stream)
