"""int8-state gated delta-rule (Gated DeltaNet) kernels for AMD MI355X (gfx950).

The compute lives in libgdnq.so (C ABI: include/gdnq.h); `ops` wraps it for
torch tensors.  Importing `ops` loads the library and fails if it is missing.
"""

__all__ = ["ops"]
