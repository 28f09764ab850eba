"""MI355X-native KroQuant activation quantizer (block Kronecker transform + MXFP4).

The compute lives in ``libkq.so`` (hand-written HIP for gfx950 behind a C ABI,
declared in ``include/kq.h``).  :mod:`.kq` is the thin ctypes binding;
:mod:`.inputs` draws the seeded synthetic workloads.
"""
