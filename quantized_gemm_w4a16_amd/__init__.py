"""MI355X (gfx950) W4A16 linear layer with a per-token gated Error Compensator.

The compute path lives in ``libspear.so`` (HIP kernels behind a C ABI declared
in ``include/spear.h``); ``quantized_gemm_w4a16_amd.spear`` is the thin ctypes
binding.  Importing this package loads nothing: the library is opened on first
use and a missing library raises.
"""
