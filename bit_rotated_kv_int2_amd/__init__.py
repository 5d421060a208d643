"""OSCAR rotated-INT2 KV decode attention for MI355X (gfx950).

The compute lives in ``liboscar.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/oscar.h``).  ``bit_rotated_kv_int2_amd.oscar`` is the thin
ctypes binding; ``synth`` holds the seeded synthetic inputs.  The shared library
is loaded on first use, so importing the package never needs a GPU.
"""
