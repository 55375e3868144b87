"""MI355X-native fused EXL3 routed-experts layer.

The compute path is the HIP library ``libexl3moe.so`` (gfx950 kernels behind a
C ABI declared in ``include/exl3moe.h``); ``trellis_quantized_moe_amd.exl3``
is its thin ctypes binding. ``synth`` draws seeded synthetic inputs.
Importing the package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
