"""MI355X (gfx950) MoE decode-layer step behind a C ABI (libkk.so, include/kk.h).

``moe_layer_skinny_amd.kk`` is the ctypes binding; the kernels are in ``csrc/``.
"""
from . import kk  # noqa: F401
